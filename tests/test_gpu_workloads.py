"""GPU path at the full workload sizes, in the configuration the benchmark times.

The default benchmark workload is also compared in full (test_default_workload_in_full).
At the larger sizes the oracle cannot run in full, so it computes sampled outputs one by
one, drawn in strata so that every tile the GPU schedules is checked at least once:
 - h: one row per (expert, 256-row tile) of the sorted positions (every row when the
   layer is small);
 - out, dx, d_topk_weights: the token of one sorted position per 256 (every token of a
   small layer), plus the first, last and busiest token;
 - dW_down: one row per (expert, 256-row tile of I); a row spans every column tile;
 - dW_up: one (gate, up) column pair per (expert, 256-column tile of 2I); a column
   spans every row tile.
Properties that hold at any size are checked on the full tensors: metadata bit-exact,
exact zeros for empty rows and experts, zeros of d_topk_weights at -1 slots.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, Gpu, assert_close, np64

pytestmark = pytest.mark.gpu

KEYS = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores"]
TILE = 256  # stratum: the row and column tile of the grouped GEMMs at these sizes


def strata(m, rng, N, I, idx):
    """Sampled rows, tokens, dW_down rows and dW_up column pairs (see module docstring)."""
    P, E = m["P"], m["E"]
    foff, freq = m["expert_frequency_offset"], m["expert_frequency"]
    h_rows = []
    for e in range(E):
        for r0 in range(int(foff[e]), int(foff[e + 1]), TILE):
            h_rows.append(int(rng.integers(r0, min(r0 + TILE, int(foff[e + 1])))))
    if P <= 4 * TILE:
        h_rows = list(range(P))
    valid_rows = (idx >= 0).sum(axis=1)
    if N <= 4 * TILE:
        toks = list(range(N))
    else:
        toks = [int(m["x_gather_idx"][int(rng.integers(s, min(s + TILE, P)))])
                for s in range(0, P, TILE)]
        toks += [0, N - 1, int(np.argmax(valid_rows))]
    toks = np.array(sorted(set(toks)), np.int64)
    dwd_e, dwd_j, dwu_e, dwu_j = [], [], [], []
    for e in np.nonzero(freq)[0]:
        for r0 in range(0, I, TILE):
            dwd_e.append(int(e))
            dwd_j.append(int(rng.integers(r0, min(r0 + TILE, I))))
        for c0 in range(0, I, TILE // 2):  # pairs (2j, 2j+1): 128 pairs per column tile
            dwu_e.append(int(e))
            dwu_j.append(int(rng.integers(c0, min(c0 + TILE // 2, I))))
    return h_rows, toks, (np.array(dwd_e), np.array(dwd_j)), (np.array(dwu_e), np.array(dwu_j))


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
    h_rows, toks, (dwd_e, dwd_j), (dwu_e, dwu_j) = strata(m, rng, N, I, idx)
    print(f"workload {name}: {len(h_rows)} h rows, {len(toks)} tokens, {len(dwd_e)} dW_down "
          f"rows, {len(dwu_e)} dW_up column pairs", flush=True)
    hs = oracle.sample_h_rows(d["x"], d["w_up"], m, h_rows)
    assert_close(np64(g.h[h_rows]), hs, tol, "h rows")
    st = oracle.sample_tokens(d["x"], d["w_up"], d["w_down"], idx, w, toks,
                              dout=d.get("dout") if cfg["backward"] else None)
    out = np64(g.out)
    valid_rows = (idx >= 0).sum(axis=1)
    assert_close(out[toks], st["out"], tol, "out rows")
    assert np.all(out[valid_rows == 0] == 0)

    if not cfg["backward"]:
        return
    assert_close(np64(g.dx)[toks], st["dx"], tol, "dx rows")
    dtw = g.dtw.cpu().numpy().astype(np.float64)
    assert_close(dtw[toks], st["d_topk_weights"], tol, "d_topk_weights rows")
    assert np.all(dtw[idx < 0] == 0)
    assert np.all(np64(g.dx)[valid_rows == 0] == 0)

    dwd = oracle.sample_dw_down_rows(d["x"], d["w_up"], d["dout"], m, dwd_e, dwd_j)
    dw_down = g.dw_down
    got_dwd = np64(dw_down[g.torch.from_numpy(dwd_e).to(dw_down.device),
                           g.torch.from_numpy(dwd_j).to(dw_down.device)])
    assert_close(got_dwd, dwd, tol, "dw_down rows")
    cols = oracle.sample_dw_up_cols(d["x"], d["w_up"], d["w_down"], d["dout"], m, dwu_e, dwu_j)
    dw_up = g.dw_up
    te = g.torch.from_numpy(dwu_e).to(dw_up.device)
    tj = g.torch.from_numpy(2 * dwu_j).to(dw_up.device)
    got_cols = np.stack([np64(dw_up[te, :, tj]), np64(dw_up[te, :, tj + 1])], axis=1)
    assert_close(got_cols, cols, tol, "dw_up columns")
    freq = m["expert_frequency"]
    for e in np.nonzero(freq == 0)[0]:
        assert np.all(np64(g.dw_up[int(e)]) == 0) and np.all(np64(g.dw_down[int(e)]) == 0)


@pytest.mark.parametrize("name", ["qwen3_rank", "dsv3_rank"])
def test_workload_bitwise_repeatable(name):
    """The whole path twice on the same inputs at the full workload size: every output
    bit for bit the same (persistent tile walks, the weight gradients' XCD mappings and
    the per-token combine take no data-dependent order)."""
    d = synth.make_inputs(name, 0, dout=True)
    print(f"workload {name}: two full runs", flush=True)
    res = []
    for _ in range(2):
        g = Gpu(d)
        g.build()
        g.forward()
        g.backward()
        g.torch.cuda.synchronize()
        res.append([t.clone() for t in (g.out, g.h, g.dx, g.dw_up, g.dw_down, g.dtw)])
        del g
    import torch
    for a, b in zip(*res):
        bits = {2: torch.int16, 4: torch.int32}[a.element_size()]
        assert torch.equal(a.contiguous().view(bits), b.contiguous().view(bits))


def test_default_workload_in_full():
    """The default benchmark workload (16384 tokens, H 2048, I 512, 32 experts, top-8,
    24717 pairs) element by element in full: every element of out, h, dx, dW_up, dW_down
    and d_topk_weights against the fp64 oracle (about 40 s of oracle time on 16 threads),
    with the weight gradients on whole experts per XCD, as the benchmark runs them."""
    from test_gpu_expert import run_case

    d = synth.make_inputs("qwen3_rank", 0, dout=True)
    run_case(d)


@pytest.mark.parametrize("n", [1024, 4096])
def test_default_dims_at_few_tokens_in_full(n):
    """The default workload's dimensions and routing at 1024 and 4096 tokens, where the
    grouped GEMMs take 128x128 tiles (fewer 256x256 tiles than CUs) and, at 1024 tokens,
    so do the weight gradients (under 128 rows per expert): every output and gradient in
    full against the fp64 oracle."""
    from test_gpu_expert import run_case

    d = synth.make_inputs(dict(synth.CONFIGS["qwen3_rank"], N=n), 0, dout=True)
    run_case(d)
