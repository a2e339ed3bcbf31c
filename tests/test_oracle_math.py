"""Pins of the oracle's forward and backward (CPU only).

What the method computes (GitHub issue #68 on Dao-AILab/sonic-moe: local expert
compute from the non-expand layout to local_out [N,H], and router-score
gradients in [N,K]; Hysen Labs page: SwiGLU with interleaved gate/up columns and
no bias) is pinned here against constructions that do not reuse the oracle's
code:
 - brute force per token and slot, independent of the metadata;
 - a dense SwiGLU MLP in numpy float64 for K=1, E=1, w=1;
 - linearity in the router weights, invariance under permuting a row's slots,
   NaN weights in -1 slots never leaking;
 - central finite differences of L = sum(out * dout) for every gradient entry;
 - dscore computed two ways, and the rank-1 closed form of dW_down;
 - the sampled entry points against the full-tensor ones.
"""
import numpy as np
import pytest

import oracle
import synth


def silu(g):
    return g / (1.0 + np.exp(-g))


def rand_case(N, H, I, E, K, seed, p_invalid=0.2, dup=False):
    rng = np.random.default_rng(seed)
    if dup:
        idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(N)]).astype(np.int32)
    idx[rng.random((N, K)) < p_invalid] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[idx < 0] = 0.0
    x = rng.standard_normal((N, H))
    wu = rng.standard_normal((E, H, 2 * I)) * 0.3
    wd = rng.standard_normal((E, I, H)) * 0.3
    dout = rng.standard_normal((N, H))
    return idx, w, x, wu, wd, dout


def run_fwd(idx, w, x, wu, wd):
    m = oracle.build_metadata(idx, w, wu.shape[0])
    return m, oracle.forward(x, wu, wd, m)


def relerr(a, b):
    s = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / s


@pytest.mark.parametrize("seed", range(6))
def test_forward_matches_bruteforce(seed):
    idx, w, x, wu, wd, _ = rand_case(7, 12, 10, 5, 3, seed, dup=(seed % 2 == 1))
    _, f = run_fwd(idx, w, x, wu, wd)
    bf = oracle.bruteforce_forward(x, idx, w, wu, wd)
    assert relerr(f["out"], bf) < 1e-12


def test_dense_mlp_special_case():
    """K=1, E=1, every slot valid, weight 1: out = (silu(x Wg) * (x Wu)) Wd with
    Wg = W_up[:, 0::2] and Wu = W_up[:, 1::2] (interleaved gate/up columns)."""
    rng = np.random.default_rng(3)
    N, H, I = 9, 16, 12
    x = rng.standard_normal((N, H))
    wu = rng.standard_normal((1, H, 2 * I)) * 0.3
    wd = rng.standard_normal((1, I, H)) * 0.3
    idx = np.zeros((N, 1), np.int32)
    w = np.ones((N, 1), np.float32)
    _, f = run_fwd(idx, w, x, wu, wd)
    ref = (silu(x @ wu[0][:, 0::2]) * (x @ wu[0][:, 1::2])) @ wd[0]
    assert relerr(f["out"], ref) < 1e-12
    assert relerr(f["h"], x @ wu[0]) < 1e-12


def test_linear_in_router_weights():
    idx, w, x, wu, wd, _ = rand_case(6, 8, 6, 4, 3, 11)
    _, f1 = run_fwd(idx, w, x, wu, wd)
    _, f2 = run_fwd(idx, (w * 4).astype(np.float32), x, wu, wd)  # exact scaling by a power of 2
    assert np.array_equal(f2["out"], 4 * f1["out"])


def test_slot_permutation_invariance():
    idx, w, x, wu, wd, _ = rand_case(6, 8, 6, 5, 4, 12)
    _, f1 = run_fwd(idx, w, x, wu, wd)
    perm = np.array([2, 0, 3, 1])
    _, f2 = run_fwd(np.ascontiguousarray(idx[:, perm]), np.ascontiguousarray(w[:, perm]), x, wu, wd)
    assert relerr(f2["out"], f1["out"]) < 1e-12


def test_invalid_slot_weights_never_leak():
    idx, w, x, wu, wd, _ = rand_case(8, 8, 6, 4, 3, 13, p_invalid=0.4)
    _, f1 = run_fwd(idx, w, x, wu, wd)
    w2 = w.copy()
    w2[idx < 0] = np.nan
    _, f2 = run_fwd(idx, w2, x, wu, wd)
    assert np.array_equal(f1["out"], f2["out"])
    w3 = w.copy()
    w3[idx < 0] = 1e4
    _, f3 = run_fwd(idx, w3, x, wu, wd)
    assert np.array_equal(f1["out"], f3["out"])


def test_empty_rows_are_exact_zero():
    idx, w, x, wu, wd, _ = rand_case(6, 8, 6, 4, 2, 14)
    idx[2] = -1
    w[2] = 0
    _, f = run_fwd(idx, w, x, wu, wd)
    assert np.all(f["out"][2] == 0.0)


def loss(idx, w, x, wu, wd, dout):
    _, f = run_fwd(idx, w, x, wu, wd)
    return float(np.sum(f["out"] * dout))


def test_backward_central_finite_differences():
    N, H, I, E, K = 4, 8, 8, 3, 2
    idx, w, x, wu, wd, dout = rand_case(N, H, I, E, K, 21, p_invalid=0.25)
    idx[:, :] = np.array([[0, 2], [1, -1], [2, 0], [-1, 1]], np.int32)
    w[idx < 0] = 0
    m, f = run_fwd(idx, w, x, wu, wd)
    g = oracle.backward(x, wu, wd, dout, m, f)
    eps = 1e-6

    def fd(arr, setter):
        out = np.zeros(arr.shape)
        for pos in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[pos] += eps
            a2 = arr.copy(); a2[pos] -= eps
            out[pos] = (setter(a1) - setter(a2)) / (2 * eps)
        return out

    gx = fd(x, lambda a: loss(idx, w, a, wu, wd, dout))
    gwu = fd(wu, lambda a: loss(idx, w, x, a, wd, dout))
    gwd = fd(wd, lambda a: loss(idx, w, x, wu, a, dout))
    assert relerr(g["dx"], gx) < 1e-6
    assert relerr(g["dw_up"], gwu) < 1e-6
    assert relerr(g["dw_down"], gwd) < 1e-6
    # router weights: the loss is linear in each weight, so a central difference
    # with a large step is exact up to rounding; use the realised fp32 step.
    gw = np.zeros((N, K))
    for t in range(N):
        for k in range(K):
            w1 = w.copy(); w1[t, k] = np.float32(w[t, k] + np.float32(0.5))
            w2 = w.copy(); w2[t, k] = np.float32(w[t, k] - np.float32(0.5))
            step = float(w1[t, k]) - float(w2[t, k])
            gw[t, k] = (loss(idx, w1, x, wu, wd, dout) - loss(idx, w2, x, wu, wd, dout)) / step
    gw[idx < 0] = 0.0
    assert relerr(g["d_topk_weights"], gw) < 1e-9
    assert np.all(g["d_topk_weights"][idx < 0] == 0.0)


def test_dscore_two_ways_and_rank1_dw_down():
    idx, w, x, wu, wd, dout = rand_case(5, 10, 6, 3, 2, 31)
    m, f = run_fwd(idx, w, x, wu, wd)
    g = oracle.backward(x, wu, wd, dout, m, f)
    # <dout[t], y[s]> == <dout[t] W_down[e]^T, a[s]>
    for q in range(m["P"]):
        t, k, e = m["pair_token"][q], m["pair_slot"][q], m["pair_expert"][q]
        s = m["s_reverse_scatter_idx"][q]
        v1 = dout[t] @ f["y"][s]
        v2 = (dout[t] @ wd[e].T) @ f["a"][s]
        assert abs(g["d_topk_weights"][t, k] - v1) <= 1e-12 * max(1, abs(v1))
        assert abs(v1 - v2) <= 1e-10 * max(1, abs(v1))
    # one token, one expert: dW_down = (w a)^T dout, rank one
    idx1 = np.array([[1]], np.int32)
    w1 = np.array([[0.625]], np.float32)
    m1, f1 = run_fwd(idx1, w1, x[:1], wu, wd)
    g1 = oracle.backward(x[:1], wu, wd, dout[:1], m1, f1)
    a = silu(x[0] @ wu[1][:, 0::2]) * (x[0] @ wu[1][:, 1::2])
    assert relerr(g1["dw_down"][1], np.outer(0.625 * a, dout[0])) < 1e-12
    assert np.all(g1["dw_down"][0] == 0) and np.all(g1["dw_down"][2] == 0)
    assert np.all(g1["dw_up"][0] == 0) and np.all(g1["dw_up"][2] == 0)


def test_sampled_entry_points_match_full():
    d = synth.case(N=40, H=32, I=24, E=6, K=3, seed=5, p_invalid=0.3)
    xb, wub, wdb, db = d["x"], d["w_up"], d["w_down"], d["dout"]
    f64 = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
    x, wu, wd, dout = f64(xb), f64(wub), f64(wdb), f64(db)
    idx, w = d["topk_idx"], d["topk_weights"]
    m, f = run_fwd(idx, w, x, wu, wd)
    g = oracle.backward(x, wu, wd, dout, m, f)
    toks = np.arange(40)
    st = oracle.sample_tokens(xb, wub, wdb, idx, w, toks, dout=db)
    assert relerr(st["out"], f["out"]) < 1e-12
    assert relerr(st["dx"], g["dx"]) < 1e-12
    assert relerr(st["d_topk_weights"], g["d_topk_weights"]) < 1e-12
    rows = np.arange(m["P"])
    assert relerr(oracle.sample_h_rows(xb, wub, m, rows), f["h"]) < 1e-12
    E, I = 6, 24
    el = np.repeat(np.arange(E), I)
    jl = np.tile(np.arange(I), E)
    dwd = oracle.sample_dw_down_rows(xb, wub, db, m, el, jl).reshape(E, I, -1)
    assert relerr(dwd, g["dw_down"]) < 1e-12
    cols = oracle.sample_dw_up_cols(xb, wub, wdb, db, m, el, jl)  # [E*I, 2, H]
    dwu = np.zeros_like(g["dw_up"])
    for r, (e, jj) in enumerate(zip(el, jl)):
        dwu[e, :, 2 * jj] = cols[r, 0]
        dwu[e, :, 2 * jj + 1] = cols[r, 1]
    assert relerr(dwu, g["dw_up"]) < 1e-12
    # fp32 inputs give the same values as fp64 copies of them
    st32 = oracle.sample_tokens(x.astype(np.float32), wu.astype(np.float32),
                                wd.astype(np.float32), idx, w, toks)
    assert relerr(st32["out"], f["out"]) < 1e-12


def test_concat_gate_up_reading():
    """The concatenated W_up layout means columns [0,I) are the gates and [I,2I) the
    ups (the Hysen Labs page on SonicMoE contrasts it with the interleaved default).
    With E=1, K=1 and unit weights the layer is a dense SwiGLU MLP; written out in
    numpy on W_up = [W_gate | W_up] it must equal the oracle fed the same weights
    reordered to interleaved columns by the test helper."""
    from _util import gateup_to_concat, gateup_to_interleaved
    rng = np.random.default_rng(31)
    N, H, I = 9, 12, 5
    x = rng.standard_normal((N, H))
    w_cat = rng.standard_normal((1, H, 2 * I)) * 0.3
    w_down = rng.standard_normal((1, I, H)) * 0.3
    g, u = x @ w_cat[0][:, :I], x @ w_cat[0][:, I:]
    want = (g / (1.0 + np.exp(-g)) * u) @ w_down[0]
    idx = np.zeros((N, 1), np.int32)
    m = oracle.build_metadata(idx, np.ones((N, 1), np.float32), 1)
    got = oracle.forward(x, gateup_to_interleaved(w_cat), w_down, m)["out"]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    w = rng.standard_normal((3, 4, 2 * I))
    assert np.array_equal(gateup_to_interleaved(gateup_to_concat(w)), w)
    assert np.array_equal(gateup_to_concat(w)[..., :I], w[..., 0::2])
