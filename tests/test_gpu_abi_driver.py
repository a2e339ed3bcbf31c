"""The C ABI from plain C++: tests/abi_gpu_driver (built by __graft_entry__.build(), linked
against libmoe.so, no Python or torch inside) builds the metadata and runs the forward and
the backward through include/moe.h alone on a seeded case written here; every output it
writes back is compared with the oracle (metadata bit for bit, tensors at the bf16
tolerance). The entry points are the three calls of issue #68's proposed integration
(metadata list, dataflow, question 4)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from _util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_gpu_driver")
META = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores"]


def bf16_file(path, shape):
    bits = np.fromfile(path, dtype=np.uint16).reshape(shape)
    return f64(bits)


@pytest.mark.parametrize("shape", [dict(N=300, H=256, I=128, E=8, K=3, seed=91),
                                   dict(N=500, H=200, I=72, E=6, K=4, seed=92)])
def test_cpp_driver_through_the_c_abi(tmp_path, shape):
    assert os.path.exists(DRIVER), "tests/abi_gpu_driver is not built: run __graft_entry__.build()"
    d = synth.case(p_invalid=0.2, **shape)
    N, H, I, E, K = d["N"], d["H"], d["I"], d["E"], d["K"]
    for name in ("x", "w_up", "w_down", "dout"):
        np.ascontiguousarray(d[name], dtype=np.uint16).tofile(tmp_path / f"{name}.bin")
    np.ascontiguousarray(d["topk_idx"], dtype=np.int32).tofile(tmp_path / "topk_idx.bin")
    np.ascontiguousarray(d["topk_weights"], dtype=np.float32).tofile(tmp_path / "topk_weights.bin")
    P = int((d["topk_idx"] >= 0).sum())
    print(f"C ABI driver: N={N} H={H} I={I} E={E} K={K} capacity={P}", flush=True)
    r = subprocess.run([DRIVER, str(tmp_path), str(N), str(H), str(I), str(E), str(K), str(P)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    m = oracle.build_metadata(d["topk_idx"], d["topk_weights"], E)
    assert int(np.fromfile(tmp_path / "status.out", dtype=np.uint32)[0]) == 0
    for k in META:
        got = np.fromfile(tmp_path / f"{k}.out", dtype=np.float32 if k == "router_scores"
                          else np.int32)
        assert np.array_equal(got, m[k].astype(got.dtype)), k

    x, wu, wd, dout = f64(d["x"]), f64(d["w_up"]), f64(d["w_down"]), f64(d["dout"])
    f = oracle.forward(x, wu, wd, m)
    g = oracle.backward(x, wu, wd, dout, m, f)
    tol = TOL["bf16"]
    assert_close(bf16_file(tmp_path / "out.out", (N, H)), f["out"], tol, "out")
    assert_close(bf16_file(tmp_path / "h.out", (P, 2 * I)), f["h"], tol, "h_save")
    assert_close(bf16_file(tmp_path / "dx.out", (N, H)), g["dx"], tol, "dx")
    assert_close(bf16_file(tmp_path / "dw_up.out", (E, H, 2 * I)), g["dw_up"], tol, "dw_up")
    assert_close(bf16_file(tmp_path / "dw_down.out", (E, I, H)), g["dw_down"], tol, "dw_down")
    dtw = np.fromfile(tmp_path / "dtw.out", dtype=np.float32).reshape(N, K).astype(np.float64)
    assert_close(dtw, g["d_topk_weights"], tol, "d_topk_weights")
