"""GPU forward/backward vs the fp64 oracle, element by element, on cases small
enough for the full-tensor oracle but spanning several 128-row/128-column tiles
with ragged tails, plus the degenerate cases of the method.

Forward: local_out [N,H] (GitHub issue #68 dataflow), and the saved h.
Backward: dx, dW_up, dW_down, and d_topk_weights in [N,K] layout (issue #68,
question 4). bf16 storage: max err <= 2e-2 * max|ref| per tensor; fp32 checking
mode: <= 1e-4 * max|ref|.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, Gpu, assert_close, f64, gateup_to_concat, np64

pytestmark = pytest.mark.gpu


def oracle_full(d):
    x, wu, wd = f64(d["x"]), f64(d["w_up"]), f64(d["w_down"])
    m = oracle.build_metadata(d["topk_idx"], d["topk_weights"], d["E"])
    f = oracle.forward(x, wu, wd, m)
    g = None
    if "dout" in d:
        g = oracle.backward(x, wu, wd, f64(d["dout"]), m, f)
    return m, f, g


def run_case(d, dtype="bf16", backward=True, capacity=None):
    print(f"case N={d['N']} H={d['H']} I={d['I']} E={d['E']} K={d['K']} dtype={dtype} "
          f"capacity={capacity}", flush=True)
    m, f, gr = oracle_full(d)
    g = Gpu(d, dtype=dtype, capacity=capacity)
    g.build()
    g.forward()
    tol = TOL[dtype]
    errs = {}
    errs["out"] = assert_close(np64(g.out), f["out"], tol, "out")
    P = m["P"]
    errs["h"] = assert_close(np64(g.h[:P]), f["h"], tol, "h_save")
    if backward:
        g.backward()
        errs["dx"] = assert_close(np64(g.dx), gr["dx"], tol, "dx")
        errs["dw_up"] = assert_close(np64(g.dw_up), gr["dw_up"], tol, "dw_up")
        errs["dw_down"] = assert_close(np64(g.dw_down), gr["dw_down"], tol, "dw_down")
        got_dtw = g.dtw.cpu().numpy().astype(np.float64)
        errs["dtw"] = assert_close(got_dtw, gr["d_topk_weights"], tol, "d_topk_weights")
        assert np.all(got_dtw[d["topk_idx"] < 0] == 0.0)
    print("relative errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return g, m


def test_tiny_forward_and_backward():
    run_case(synth.make_inputs("tiny", 0))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("seed", [0, 1])
def test_medium_ragged(dtype, seed):
    # ~350 rows per expert: 3 row tiles with a ragged tail; H=384, I=256 span 3 and 2 column tiles
    d = synth.case(N=600, H=384, I=256, E=5, K=4, seed=seed, p_invalid=0.3)
    run_case(d, dtype=dtype)


def test_exact_tile_boundaries():
    # experts with 0, 127, 128, 129, 256 and 1 rows (K=1 so every row is one pair)
    sizes = [0, 127, 128, 129, 256, 1]
    idx = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])
    rng = np.random.default_rng(4)
    idx = idx[rng.permutation(idx.shape[0])][:, None]
    d = synth.case(N=idx.shape[0], H=256, I=128, E=len(sizes), K=1, seed=4, topk_idx=idx)
    g, m = run_case(d)
    assert np.all(np64(g.dw_up)[0] == 0) and np.all(np64(g.dw_down)[0] == 0)


def test_more_tiles_than_workgroups():
    """~9000 rows per expert: every grouped GEMM has more 256-row tiles than the chip holds
    workgroups at once, so each persistent workgroup walks several tiles (next-tile loads
    issued before an epilogue), each expert ending in a ragged tile."""
    d = synth.case(N=10000, H=256, I=256, E=8, K=8, seed=7, p_invalid=0.1)
    gi, _ = run_case(d)
    # the concatenated W_up layout takes the same tile walk: bit-equal to the interleaved
    # run wherever the concatenated-layout test requires it
    gc = Gpu(d, layout=1)
    gc.build()
    gc.forward()
    gc.backward()
    for a, b in [(gi.out, gc.out), (gi.h, gc.h), (gi.dw_down, gc.dw_down), (gi.dtw, gc.dtw)]:
        assert np.array_equal(np64(a), np64(b))
    assert np.array_equal(gateup_to_concat(np64(gi.dw_up)), np64(gc.dw_up))


@pytest.mark.parametrize("N,K", [(2000, 8), (24000, 8), (400, 64)])
def test_max_experts(N, K):
    """E = 1024 local experts (the largest the library takes) and K up to 64: the tile
    tables, the tile-to-expert search and the weight gradients' expert ordering at their
    largest; about 14 rows per expert (32-row tiles), about 170 (256-row tiles), and 64
    slots per token."""
    run_case(synth.case(N=N, H=128, I=128, E=1024, K=K, seed=31, p_invalid=0.1))


def test_duplicate_experts_in_a_row_and_empty_rows():
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 3, size=(200, 4)).astype(np.int32)
    idx[rng.random((200, 4)) < 0.3] = -1
    idx[7] = -1
    idx[8] = 2
    d = synth.case(N=200, H=128, I=128, E=3, K=4, seed=5, topk_idx=idx)
    g, _ = run_case(d)
    assert np.all(np64(g.out)[7] == 0) and np.all(np64(g.dx)[7] == 0)


def test_single_expert_k1():
    d = synth.case(N=300, H=256, I=256, E=1, K=1, seed=6, p_invalid=0.0)
    run_case(d)


def test_all_invalid():
    idx = -np.ones((64, 4), np.int32)
    d = synth.case(N=64, H=128, I=128, E=4, K=4, seed=7, topk_idx=idx)
    g, _ = run_case(d)
    assert np.all(np64(g.out) == 0) and np.all(np64(g.dw_up) == 0)


def test_capacity_above_P():
    d = synth.case(N=300, H=256, I=128, E=6, K=3, seed=8)
    run_case(d, capacity=300 * 3)


def test_over_capacity_writes_zeros():
    d = synth.case(N=300, H=256, I=128, E=6, K=3, seed=9)
    P = int((d["topk_idx"] >= 0).sum())
    g = Gpu(d, capacity=P - 10)
    g.build()
    g.forward()
    g.backward()
    assert g.meta_numpy()["status"] == 2
    for t in (g.out, g.dx, g.dw_up, g.dw_down, g.dtw):
        assert np.all(np64(t) == 0)


def test_poisoned_invalid_slot_weights():
    d = synth.case(N=256, H=128, I=128, E=4, K=4, seed=10, p_invalid=0.4)
    g0, _ = run_case(d, backward=True)
    d2 = dict(d)
    w = d["topk_weights"].copy()
    w[d["topk_idx"] < 0] = np.nan
    d2["topk_weights"] = w
    g1 = Gpu(d2)
    g1.build()
    g1.forward()
    g1.backward()
    for a, b in [(g0.out, g1.out), (g0.dx, g1.dx), (g0.dw_up, g1.dw_up), (g0.dtw, g1.dtw)]:
        assert np.array_equal(np64(a), np64(b))


def test_deterministic():
    d = synth.case(N=800, H=256, I=256, E=8, K=4, seed=11)
    res = []
    for _ in range(2):
        g = Gpu(d)
        g.build()
        g.forward()
        g.backward()
        res.append([np64(t) for t in (g.out, g.h, g.dx, g.dw_up, g.dw_down, g.dtw)])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_n_zero():
    d = synth.case(N=0, H=128, I=128, E=4, K=2, seed=12)
    g = Gpu(d)
    g.build()
    g.forward()
    g.backward()
    assert np.all(np64(g.dw_up) == 0) and np.all(np64(g.dw_down) == 0)


CONCAT_CASES = {
    "tiles256": dict(N=600, H=384, I=256, E=5, K=4, seed=21, p_invalid=0.3),
    # at most 16 rows per expert on average: the 32-row tiles of the up projection
    # and of the dSwiGLU backward, in both gate/up orders
    "rows32": dict(N=96, H=256, I=256, E=16, K=2, seed=22, p_invalid=0.1),
}


@pytest.mark.parametrize("shape", list(CONCAT_CASES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_concat_gate_up_layout(dtype, shape):
    """W_up stored [gates | ups] (MOE_GATEUP_CONCAT): the same layer as the interleaved
    storage of the same weights (the Hysen Labs page on SonicMoE, gate/up formats).
    Against the oracle, with dW_up compared in the concatenated order; against the
    interleaved run, the up-projection tiles hold the same values, so the forward and
    every gradient except dx (whose 2I contraction runs in another order) match bit for bit."""
    d = synth.case(**CONCAT_CASES[shape])
    print(f"concat layout case {shape} dtype={dtype}", flush=True)
    m, f, gr = oracle_full(d)
    gi = Gpu(d, dtype=dtype)
    gc = Gpu(d, dtype=dtype, layout=1)
    for g in (gi, gc):
        g.build()
        g.forward()
        g.backward()
    tol = TOL[dtype]
    assert_close(np64(gc.out), f["out"], tol, "out")
    assert_close(np64(gc.h[:m["P"]]), f["h"], tol, "h_save (interleaved)")
    assert_close(np64(gc.dx), gr["dx"], tol, "dx")
    assert_close(np64(gc.dw_up), gateup_to_concat(gr["dw_up"]), tol, "dw_up (concat)")
    assert_close(np64(gc.dw_down), gr["dw_down"], tol, "dw_down")
    assert_close(gc.dtw.cpu().numpy().astype(np.float64), gr["d_topk_weights"], tol, "dtw")
    for a, b in [(gi.out, gc.out), (gi.h, gc.h), (gi.dw_down, gc.dw_down), (gi.dtw, gc.dtw)]:
        assert np.array_equal(np64(a), np64(b))
    assert np.array_equal(gateup_to_concat(np64(gi.dw_up)), np64(gc.dw_up))


@pytest.mark.parametrize("N", [4095, 4096])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_combine_token_count_threshold(dtype, N):
    """Either side of the token count below which the combine cuts each row into column
    blocks of 64 chunks, one wavefront each (4096 tokens); H = 136 leaves a partial
    block, and rows span one or several blocks in the two dtypes."""
    run_case(synth.case(N=N, H=136, I=128, E=6, K=3, seed=N, p_invalid=0.2), dtype=dtype)
