"""Decode-sized forwards (a few rows per expert, bf16): the 32-row tiles of two wavefronts
that stream the active experts' weights where H and I fill 128-wide tiles, the partial-tile
kernels otherwise. Full tensors against the fp64 oracle (out, the
saved h, and the backward that consumes that h), both gate/up orders, ragged H and I, an
expert holding most of the rows, capacity above and below P, and the decode workload
itself (N = 8, H = 7168, I = 2048, 32 experts, top-8) element by element.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, Gpu, assert_close, f64, gateup_to_concat, np64
from test_gpu_expert import oracle_full, run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,I", [(256, 128), (2048, 1024), (200, 72)])
def test_decode_sized_forward_and_backward(H, I):
    # 8 tokens x 8 slots over 32 experts with 10 % invalid: P <= 64 = 2E
    run_case(synth.case(N=8, H=H, I=I, E=32, K=8, seed=H + I, p_invalid=0.1))


def test_decode_sized_concat_layout():
    d = synth.case(N=8, H=256, I=128, E=32, K=8, seed=61, p_invalid=0.1)
    m, f, gr = oracle_full(d)
    gi, gc = Gpu(d), Gpu(d, layout=1)
    for g in (gi, gc):
        g.build()
        g.forward()
        g.backward()
    tol = TOL["bf16"]
    assert_close(np64(gc.out), f["out"], tol, "out")
    assert_close(np64(gc.h[:m["P"]]), f["h"], tol, "h_save (interleaved)")
    assert_close(np64(gc.dw_up), gateup_to_concat(gr["dw_up"]), tol, "dw_up (concat)")
    # the same tiles in the other column order: the forward is bit-identical
    assert np.array_equal(np64(gi.out), np64(gc.out))
    assert np.array_equal(np64(gi.h), np64(gc.h))


def test_decode_sized_expert_with_many_rows():
    """One expert holds 21 rows and another about ten, the others one or none; capacity
    64, above P."""
    N, K, E = 32, 2, 32
    rng = np.random.default_rng(62)
    idx = -np.ones((N, K), np.int32)
    idx[:21, 0] = 5
    idx[21:, 0] = rng.choice(np.arange(6, 32), size=N - 21, replace=False)
    idx[rng.random(N) < 0.3, 1] = 3
    d = synth.case(N=N, H=264, I=200, E=E, K=K, seed=62, topk_idx=idx)
    run_case(d, capacity=2 * E)


def test_decode_sized_over_capacity_writes_zeros():
    d = synth.case(N=8, H=256, I=136, E=32, K=8, seed=63, p_invalid=0.1)
    P = int((d["topk_idx"] >= 0).sum())
    g = Gpu(d, capacity=P - 3)
    g.build()
    g.forward()
    assert g.meta_numpy()["status"] == 2
    assert np.all(np64(g.out) == 0)


def test_decode_workload_full_forward():
    """The decode workload at its full size: every element of out and h."""
    d = synth.make_inputs("decode", 0, dout=False)
    print(f"decode workload N={d['N']} H={d['H']} I={d['I']} E={d['E']} K={d['K']}", flush=True)
    x, wu, wd = f64(d["x"]), f64(d["w_up"]), f64(d["w_down"])
    m = oracle.build_metadata(d["topk_idx"], d["topk_weights"], d["E"])
    f = oracle.forward(x, wu, wd, m)
    g = Gpu(d)
    g.build()
    g.forward()
    tol = TOL["bf16"]
    assert_close(np64(g.out), f["out"], tol, "out")
    assert_close(np64(g.h[:m["P"]]), f["h"], tol, "h_save")
