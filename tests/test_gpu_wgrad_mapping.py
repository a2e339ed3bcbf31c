"""The weight-gradient GEMMs' two tile-to-XCD mappings, each against the fp64 oracle on
full tensors (forward and backward, bf16). The kernel decides on the device from the
segment offsets: with E a multiple of 8 and the experts' row counts even enough that
dealing them to the 8 XCDs in a snake (largest first: 0..7, then 7..0, ...) leaves no XCD
more than 1/32 above the mean, each XCD takes whole experts; otherwise each XCD takes a
rectangle of every expert's tiles. The host reproduces that decision here so that each
case is known to exercise the mapping it names (weight gradients are the dW of issue #68,
question 4: correct in the [N_recv, K] layout).
"""
import numpy as np
import pytest

import synth
from _util import np64
from test_gpu_expert import run_case

pytestmark = pytest.mark.gpu


def takes_whole_experts(d):
    E = d["E"]
    idx = d["topk_idx"]
    cnt = np.bincount(idx[(idx >= 0) & (idx < E)].ravel(), minlength=E).astype(np.int64)
    if E % 8:
        return False
    # descending by count, ties by the lower expert id
    order = sorted(range(E), key=lambda e: (-cnt[e], e))
    tot = np.zeros(8, np.int64)
    for r in range(E // 8):
        for x in range(8):
            tot[x] += cnt[order[r * 8 + (7 - x if r % 2 else x)]]
    return tot.max() * 8 * 32 <= tot.sum() * 33


def skewed(N, E, K, seed, heavy=3, share=0.5):
    """Uniform routing, then about `share` of the tokens' first slot sent to one expert."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(N)]).astype(np.int32)
    sel = rng.random(N) < share
    for t in np.nonzero(sel)[0]:
        if heavy not in idx[t]:
            idx[t, 0] = heavy
    return idx


@pytest.mark.parametrize("H,I", [(256, 128), (200, 72)])
def test_whole_experts_per_xcd(H, I):
    # 16 experts of about 750 rows each: the snake deals two per XCD almost evenly
    d = synth.case(N=3000, H=H, I=I, E=16, K=4, seed=81, p_invalid=0.0)
    assert takes_whole_experts(d)
    run_case(d)


def test_whole_experts_per_xcd_four_rounds():
    # 32 experts, four per XCD one after another, with the 256-wide tiles (H, I multiples
    # of 256 and 128) and several row-tile groups per expert
    d = synth.case(N=4000, H=1024, I=256, E=32, K=4, seed=82, p_invalid=0.0)
    assert takes_whole_experts(d)
    run_case(d)


@pytest.mark.parametrize("H,I", [(256, 128), (200, 72)])
def test_rectangles_when_skewed(H, I):
    N, E, K = 3000, 16, 4
    d = synth.case(N=N, H=H, I=I, E=E, K=K, seed=83, topk_idx=skewed(N, E, K, 83))
    assert not takes_whole_experts(d)
    run_case(d)


def test_rectangles_when_experts_not_a_multiple_of_8():
    d = synth.case(N=2000, H=256, I=128, E=12, K=4, seed=84, p_invalid=0.0)
    assert not takes_whole_experts(d)
    run_case(d)


def test_whole_experts_per_xcd_all_empty():
    """Every slot invalid with 16 experts: the XCD totals are all zero, so the whole-expert
    mapping is taken, and every expert's gradient must still be written as exact zeros."""
    N, E, K = 300, 16, 4
    d = synth.case(N=N, H=256, I=128, E=E, K=K, seed=85, topk_idx=-np.ones((N, K), np.int32))
    assert takes_whole_experts(d)
    g, _ = run_case(d)
    assert np.all(np64(g.dw_up) == 0) and np.all(np64(g.dw_down) == 0)
