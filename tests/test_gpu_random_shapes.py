"""Seeded random shapes through the whole layer (metadata, forward, backward), every
element against the fp64 oracle: hidden and intermediate sizes any multiple of 8 (so
both the 256-wide and the edge-bounded tiles, and in the weight gradients both XCD
mappings, are drawn), 1 to 64 experts, top-1 to top-8, invalid slots, capacities above
and below the pair count, bf16 and the fp32 checking mode, both gate/up layouts, and
decode-sized batches (the 32-row tiles). The draws are fixed by the case number, so a
failure names a reproducible case (issue #68, question 4: forward and backward right in
the [N_recv, K] layout at any shape).
"""
import numpy as np
import pytest

import synth
from _util import TOL, Gpu, assert_close, gateup_to_concat, np64
from test_gpu_expert import oracle_full

pytestmark = pytest.mark.gpu

CASES = 24


def draw(case):
    rng = np.random.default_rng(1000 + case)
    E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24, 32, 40, 64]))
    K = int(rng.integers(1, min(E, 6) + 1))
    N = int(rng.integers(1, 1500))
    if case % 4 == 0:
        N = 1200 + int(rng.integers(0, 300))  # several row tiles per expert
    H = 8 * int(rng.integers(1, 65))
    I = 8 * int(rng.integers(1, 49))
    if case % 3 == 0:  # whole 256-wide tiles in the forward and weight gradients
        H = 256 * int(rng.integers(1, 3))
        I = 128 * int(rng.integers(1, 4))
    if case % 8 == 5:  # decode-sized: the 32-row tiles that stream the experts' weights
        E, K = 32, 8
        N = int(rng.integers(2, 60))
        H = 128 * int(rng.integers(1, 5))
        I = 64 * int(rng.integers(1, 6))
    p_invalid = float(rng.choice([0.0, 0.1, 0.3]))
    dtype = "fp32" if case % 3 == 1 else "bf16"
    layout = int(case % 2)
    cap = str(rng.choice(["exact", "exact", "above", "above", "below"]))
    if case % 8 == 5:  # the 32-row tiles are bf16 kernels; compare their outputs
        dtype, cap = "bf16", ("above" if case % 16 == 5 else "exact")
    return dict(N=N, H=H, I=I, E=E, K=K, p_invalid=p_invalid, dtype=dtype, layout=layout,
                cap=cap, seed=2000 + case)


@pytest.mark.parametrize("case", range(CASES))
def test_random_shape(case):
    c = draw(case)
    d = synth.case(N=c["N"], H=c["H"], I=c["I"], E=c["E"], K=c["K"], seed=c["seed"],
                   p_invalid=c["p_invalid"])
    P = int(((d["topk_idx"] >= 0) & (d["topk_idx"] < c["E"])).sum())
    capacity = None
    if c["cap"] == "above":
        capacity = P + 1 + case
    elif c["cap"] == "below" and P > 0:
        capacity = max(0, P - 1 - case)
    print(f"random case {case}: {c} P={P} capacity={capacity}", flush=True)
    g = Gpu(d, dtype=c["dtype"], capacity=capacity, layout=c["layout"])
    g.build()
    g.forward()
    g.backward()
    g.torch.cuda.synchronize()
    meta = g.meta_numpy()
    assert meta["P"] == P
    if capacity is not None and capacity < P:
        # over capacity: status bit 2 and zeros in every output and gradient
        assert meta["status"] == 2
        for name, t in [("out", g.out), ("dx", g.dx), ("dw_up", g.dw_up),
                        ("dw_down", g.dw_down), ("dtw", g.dtw)]:
            assert np.all(np64(t) == 0), name
        return
    assert meta["status"] == 0
    m, f, gr = oracle_full(d)
    tol = TOL[c["dtype"]]
    assert_close(np64(g.out), f["out"], tol, "out")
    assert_close(np64(g.h[:P]), f["h"], tol, "h_save")
    assert_close(np64(g.dx), gr["dx"], tol, "dx")
    dwu = gr["dw_up"] if c["layout"] == 0 else gateup_to_concat(gr["dw_up"])
    assert_close(np64(g.dw_up), dwu, tol, "dw_up")
    assert_close(np64(g.dw_down), gr["dw_down"], tol, "dw_down")
    dtw = g.dtw.cpu().numpy().astype(np.float64)
    assert_close(dtw, gr["d_topk_weights"], tol, "d_topk_weights")
    assert np.all(dtw[d["topk_idx"] < 0] == 0)
