"""GPU path at the full workload sizes, in the configuration the benchmark times.

The oracle cannot run these sizes in full, so it computes sampled outputs one
by one (whole rows of out, dx, d_topk_weights for sampled tokens; rows of h;
rows of dW_down and column pairs of dW_up for sampled experts, including the
largest and an empty one), and properties that hold at any size are checked on
the full tensors: metadata bit-exact, exact zeros for empty rows and experts,
zeros of d_topk_weights at -1 slots.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, Gpu, assert_close, np64

pytestmark = pytest.mark.gpu

KEYS = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores"]


@pytest.mark.parametrize("name", ["qwen3_rank", "dsv3_rank", "decode", "long_prefill"])
def test_workload(name):
    cfg = synth.CONFIGS[name]
    print(f"workload {name}: generating inputs", flush=True)
    d = synth.make_inputs(name, 0, dout=cfg["backward"])
    idx, w = d["topk_idx"], d["topk_weights"]
    N, K, E, H, I = d["N"], d["K"], d["E"], d["H"], d["I"]
    tol = TOL["bf16"]
    g = Gpu(d)
    print(f"workload {name}: N={N} H={H} I={I} E={E} K={K} P={g.P}", flush=True)
    g.build()
    g.forward()
    if cfg["backward"]:
        g.backward()
    g.torch.cuda.synchronize()
    print(f"workload {name}: GPU done, checking", flush=True)

    # metadata: bit-exact in full
    m = oracle.build_metadata(idx, w, E)
    got = g.meta_numpy()
    assert got["status"] == 0
    for k in KEYS:
        assert np.array_equal(got[k], m[k].astype(got[k].dtype)), k

    rng = np.random.default_rng(1)
    valid_rows = ((idx >= 0).sum(axis=1))
    toks = sorted(set([0, N - 1, int(np.argmax(valid_rows))] +
                      rng.choice(N, size=min(N, 9), replace=False).tolist()))
    toks = np.array(toks, np.int64)
    st = oracle.sample_tokens(d["x"], d["w_up"], d["w_down"], idx, w, toks,
                              dout=d.get("dout") if cfg["backward"] else None)
    out = np64(g.out)
    assert_close(out[toks], st["out"], tol, "out rows")
    assert np.all(out[valid_rows == 0] == 0)

    freq = m["expert_frequency"]
    foff = m["expert_frequency_offset"]
    big = int(np.argmax(freq))
    rows = sorted(set([0, int(foff[big]), int(foff[big + 1]) - 1, m["P"] - 1] +
                      rng.choice(m["P"], size=4, replace=False).tolist()))
    hs = oracle.sample_h_rows(d["x"], d["w_up"], m, rows)
    assert_close(np64(g.h[rows]), hs, tol, "h rows")

    if not cfg["backward"]:
        return
    assert_close(np64(g.dx)[toks], st["dx"], tol, "dx rows")
    dtw = g.dtw.cpu().numpy().astype(np.float64)
    assert_close(dtw[toks], st["d_topk_weights"], tol, "d_topk_weights rows")
    assert np.all(dtw[idx < 0] == 0)
    assert np.all(np64(g.dx)[valid_rows == 0] == 0)

    nz = np.nonzero(freq)[0]
    small = int(nz[np.argmin(freq[nz])])
    experts = sorted(set([big, small, int(rng.choice(nz))]))
    el = np.repeat(experts, 2)
    jl = rng.integers(0, I, size=el.shape[0])
    dwd = oracle.sample_dw_down_rows(d["x"], d["w_up"], d["dout"], m, el, jl)
    got_dwd = np.stack([np64(g.dw_down[int(e), int(j)]) for e, j in zip(el, jl)])
    assert_close(got_dwd, dwd, tol, "dw_down rows")
    cols = oracle.sample_dw_up_cols(d["x"], d["w_up"], d["w_down"], d["dout"], m, el, jl)
    got_cols = np.stack([np.stack([np64(g.dw_up[int(e), :, 2 * int(j)]),
                                   np64(g.dw_up[int(e), :, 2 * int(j) + 1])])
                         for e, j in zip(el, jl)])
    assert_close(got_cols, cols, tol, "dw_up columns")
    for e in np.nonzero(freq == 0)[0]:
        assert np.all(np64(g.dw_up[int(e)]) == 0) and np.all(np64(g.dw_down[int(e)]) == 0)
