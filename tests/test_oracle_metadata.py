"""Pins of the oracle's routing metadata (CPU only).

The metadata's names come from GitHub issue #68 on Dao-AILab/sonic-moe (the list
of arrays SonicMoE's grouped GEMM needs). With the readings the oracle documents
(token-major pair order with ascending slot inside a token; stable sort by
expert), the answer is unique, so it is pinned by:
 - an independent construction: numpy's stable argsort of the expert ids of the
   pair list (a textbook routine, different code from the oracle's counting sort);
 - invariants that hold for any input;
 - exhaustive enumeration of every topk_idx over {-1..E-1} for tiny N, K, E.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402


def reference_by_stable_argsort(idx: np.ndarray, w: np.ndarray, E: int) -> dict:
    N, K = idx.shape
    valid = (idx >= 0) & (idx < E)
    t, k = np.nonzero(valid)            # row-major: token-major, ascending slot
    pe = idx[t, k]
    P = t.shape[0]
    perm = np.argsort(pe, kind="stable")  # sorted position s -> pair q
    inv = np.empty(P, np.int64)
    inv[perm] = np.arange(P)
    freq = np.bincount(pe, minlength=E)
    rows = valid.sum(axis=1)
    return dict(
        P=P,
        expert_frequency=freq,
        expert_frequency_offset=np.concatenate([[0], np.cumsum(freq)]),
        x_gather_idx=t[perm],
        s_scatter_idx=perm,
        s_reverse_scatter_idx=inv,
        num_activated_expert_per_token_offset=np.concatenate([[0], np.cumsum(rows)]),
        router_scores=w[t, k],
        pair_token=t, pair_slot=k, pair_expert=pe,
    )


KEYS = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores",
        "pair_token", "pair_slot", "pair_expert"]


def assert_same(m, r):
    assert m["P"] == r["P"]
    for key in KEYS:
        a, b = np.asarray(m[key]), np.asarray(r[key])
        assert a.shape == b.shape, key
        assert np.array_equal(a, b.astype(a.dtype)), key


def check_invariants(m, idx, E):
    P = m["P"]
    freq, foff = m["expert_frequency"], m["expert_frequency_offset"]
    toff = m["num_activated_expert_per_token_offset"]
    xg, ss, sr = m["x_gather_idx"], m["s_scatter_idx"], m["s_reverse_scatter_idx"]
    N, K = idx.shape
    assert freq.sum() == P == foff[E] == toff[N]
    assert foff[0] == 0 and toff[0] == 0
    assert np.array_equal(np.diff(foff), freq)
    assert np.array_equal(np.diff(toff), ((idx >= 0) & (idx < E)).sum(axis=1))
    # s_scatter and s_reverse are mutually inverse permutations of [0,P)
    assert np.array_equal(np.sort(ss), np.arange(P))
    assert np.array_equal(ss[sr], np.arange(P))
    assert np.array_equal(sr[ss], np.arange(P))
    # the gather index of a pair's sorted position is the pair's token
    assert np.array_equal(xg[sr], m["pair_token"])
    # each expert segment holds only that expert, with strictly increasing q
    for e in range(E):
        seg = ss[foff[e]:foff[e + 1]]
        assert np.all(m["pair_expert"][seg] == e)
        assert np.all(np.diff(seg) > 0)
    # -1 slots appear nowhere: every pair's slot is valid
    if P:
        assert np.all(idx[m["pair_token"], m["pair_slot"]] >= 0)


def test_exhaustive_tiny():
    """Every topk_idx in {-1..E-1}^(N*K) for N<=3, K<=2, E<=3."""
    count = 0
    for N, K, E in [(1, 1, 1), (2, 1, 2), (3, 2, 3), (2, 2, 3), (3, 1, 3), (1, 2, 2)]:
        for vals in itertools.product(range(-1, E), repeat=N * K):
            idx = np.array(vals, np.int32).reshape(N, K)
            w = (np.arange(N * K, dtype=np.float32).reshape(N, K) + 1) / 8
            m = oracle.build_metadata(idx, w, E)
            assert_same(m, reference_by_stable_argsort(idx, w, E))
            check_invariants(m, idx, E)
            assert m["flags"] == 0
            count += 1
    assert count > 4096


@settings(max_examples=200, deadline=None)
@given(N=st.integers(0, 40), K=st.integers(1, 9), E=st.integers(1, 20),
       p=st.floats(0.0, 1.0), seed=st.integers(0, 2**31 - 1))
def test_random_shapes(N, K, E, p, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)  # duplicates in a row allowed
    idx[rng.random((N, K)) < p] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    m = oracle.build_metadata(idx, w, E)
    assert_same(m, reference_by_stable_argsort(idx, w, E))
    check_invariants(m, idx, E)


def test_workload_routings():
    for name in ["tiny", "decode", "qwen3_rank"]:
        idx, seed = synth.make_routing(name, 0)
        E = synth.CONFIGS[name]["E"]
        w = synth.make_topk_weights(idx, seed)
        m = oracle.build_metadata(idx, w, E)
        assert_same(m, reference_by_stable_argsort(idx, w, E))
        check_invariants(m, idx, E)


def test_bad_expert_ids_flagged_and_skipped():
    idx = np.array([[0, 5], [-2, 1], [2, -1]], np.int32)
    w = np.ones((3, 2), np.float32)
    m = oracle.build_metadata(idx, w, 3)
    assert m["flags"] & oracle.FLAG_BAD_EXPERT
    clean = np.where((idx >= 0) & (idx < 3), idx, -1).astype(np.int32)
    r = reference_by_stable_argsort(clean, w, 3)
    assert_same(m, r)


def test_empty_and_all_invalid():
    for N, K in [(0, 4), (5, 3)]:
        idx = -np.ones((N, K), np.int32)
        m = oracle.build_metadata(idx, np.zeros((N, K), np.float32), 4)
        assert m["P"] == 0
        assert np.all(m["expert_frequency"] == 0)
        assert np.all(m["expert_frequency_offset"] == 0)
        assert np.all(m["num_activated_expert_per_token_offset"] == 0)


def test_hand_example():
    """A 3x2 case worked out by hand from the definitions:
    pairs q: (t0,k0,e1) (t1,k0,e0) (t1,k1,e1) (t2,k0,e2) (t2,k1,e0)."""
    idx = np.array([[1, -1], [0, 1], [2, 0]], np.int32)
    w = np.array([[0.5, 0.0], [0.25, 0.75], [0.125, 0.875]], np.float32)
    m = oracle.build_metadata(idx, w, 3)
    assert m["P"] == 5
    assert m["expert_frequency"].tolist() == [2, 2, 1]
    assert m["expert_frequency_offset"].tolist() == [0, 2, 4, 5]
    # expert 0 gets q=1,4; expert 1 gets q=0,2; expert 2 gets q=3
    assert m["s_scatter_idx"].tolist() == [1, 4, 0, 2, 3]
    assert m["x_gather_idx"].tolist() == [1, 2, 0, 1, 2]
    assert m["s_reverse_scatter_idx"].tolist() == [2, 0, 3, 4, 1]
    assert m["num_activated_expert_per_token_offset"].tolist() == [0, 1, 3, 5]
    assert m["router_scores"].tolist() == [0.5, 0.25, 0.75, 0.125, 0.875]
