"""GPU routing metadata vs the oracle: bit-exact on every workload and edge case.

The seven arrays are the ones GitHub issue #68 on Dao-AILab/sonic-moe lists; with
token-major pairs and a stable sort by expert they are unique, so the HIP path
must reproduce the oracle exactly (integer work: bit-exact; router_scores are
copies of fp32 inputs: bit-exact too).
"""
import numpy as np
import pytest

import oracle
import synth
from _util import Gpu

pytestmark = pytest.mark.gpu

KEYS = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores"]
PAIR_KEYS = {"x_gather_idx", "s_scatter_idx", "s_reverse_scatter_idx", "router_scores"}


def check(idx, w, E, capacity=None, expect_status=0):
    N, K = idx.shape
    d = dict(N=N, H=128, I=128, E=E, K=K, topk_idx=np.ascontiguousarray(idx, np.int32),
             topk_weights=np.ascontiguousarray(w, np.float32),
             x=np.zeros((N, 128), np.uint16), w_up=np.zeros((E, 128, 256), np.uint16),
             w_down=np.zeros((E, 128, 128), np.uint16))
    print(f"metadata case N={N} K={K} E={E} capacity={capacity}", flush=True)
    g = Gpu(d, capacity=capacity)
    g.build()
    got = g.meta_numpy()
    ref = oracle.build_metadata(idx, w, E)
    assert got["P"] == ref["P"]
    n = min(ref["P"], g.meta.capacity)
    for k in KEYS:
        r = ref[k]
        if k in PAIR_KEYS:  # entries at positions >= capacity are dropped
            r = r[:n]
        a = got[k]
        assert a.shape == r.shape, k
        assert np.array_equal(a, r.astype(a.dtype)), f"{k} differs"
    assert got["status"] == expect_status
    return got


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workloads(name):
    idx, seed = synth.make_routing(name, 0)
    w = synth.make_topk_weights(idx, seed)
    check(idx, w, synth.CONFIGS[name]["E"])


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("N,K,E,p", [(1, 1, 1, 0.0), (3, 2, 3, 0.3), (1000, 8, 64, 0.5),
                                     (4097, 6, 17, 0.2), (2048, 1, 1, 0.1),
                                     (3000, 16, 1024, 0.0), (50000, 3, 5, 0.9),
                                     (2000, 64, 1024, 0.2), (500, 64, 3, 0.0)])
def test_random(N, K, E, p, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)  # duplicates in a row allowed
    idx[rng.random((N, K)) < p] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    check(idx, w, E)


def test_all_invalid_and_empty():
    check(-np.ones((100, 4), np.int32), np.zeros((100, 4), np.float32), 8)
    check(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32), 8)


def test_capacity_larger_than_P():
    idx, seed = synth.make_routing("tiny", 0)
    w = synth.make_topk_weights(idx, seed)
    check(idx, w, 8, capacity=idx.size)


def test_over_capacity_sets_status():
    idx, seed = synth.make_routing("tiny", 0)
    w = synth.make_topk_weights(idx, seed)
    P = int((idx >= 0).sum())
    check(idx, w, 8, capacity=P - 7, expect_status=2)


def test_bad_expert_ids_set_status():
    rng = np.random.default_rng(9)
    idx = rng.integers(-1, 8, size=(300, 4)).astype(np.int32)
    idx[5, 1] = 8
    idx[17, 0] = -3
    w = rng.standard_normal((300, 4)).astype(np.float32)
    got = check(np.where((idx >= -1) & (idx < 8), idx, -1), w, 8)
    # the same input with the bad ids: treated as -1, flagged
    N, K = idx.shape
    d = dict(N=N, H=128, I=128, E=8, K=K, topk_idx=idx, topk_weights=w,
             x=np.zeros((N, 128), np.uint16), w_up=np.zeros((8, 128, 256), np.uint16),
             w_down=np.zeros((8, 128, 128), np.uint16))
    g = Gpu(d, capacity=got["P"])
    g.build()
    bad = g.meta_numpy()
    assert bad["status"] == 1
    for k in KEYS:
        assert np.array_equal(bad[k], got[k]), k


@pytest.mark.parametrize("N,K,E", [(300000, 8, 64), (2200000, 1, 7), (140000, 16, 1024),
                                   (600000, 8, 64), (300000, 16, 1024), (1100000, 8, 64),
                                   (8400000, 1, 7), (560000, 16, 1024)])
def test_long_columns_two_pass_scan(N, K, E):
    """Long count columns. From 2048 up to 4096 chunks (of 1024 slots at the first three
    sizes, of 2048 at the next two) one scan pass with 16 chunks per thread; beyond 4096
    chunks (the last three, 4102 to 4375 chunks of 2048 slots) the column scan runs in
    segments: a pass of segment sums, then the segments with their bases."""
    rng = np.random.default_rng(N + K + E)
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    idx[rng.random((N, K)) < 0.25] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    check(idx, w, E)


@pytest.mark.parametrize("NK", [(1 << 18) - 1, 1 << 18, (1 << 18) + 1,
                                (1 << 20) - 1, 1 << 20, (1 << 20) + 1,
                                (1 << 22) - 1, 1 << 22, (1 << 22) + 1])
def test_slot_count_thresholds(NK):
    """Either side of the slot counts where the scatter starts staging its sorted writes
    in LDS (2^18) and where the chunks grow from 512 to 1024 slots (2^20) and to 2048
    (2^22); K = 1 so that every slot count is reachable, with a ragged last chunk."""
    rng = np.random.default_rng(NK)
    E = 48
    idx = rng.integers(0, E, size=(NK, 1)).astype(np.int32)
    idx[rng.random((NK, 1)) < 0.2] = -1
    w = rng.standard_normal((NK, 1)).astype(np.float32)
    check(idx, w, E)


@pytest.mark.parametrize("NK,E", [((1 << 21) - 1, 64), (1 << 21, 64), ((1 << 21) - 1, 300),
                                  ((1 << 21) - 1, 256), (4000, 256), (4000, 257)])
def test_ranking_form_thresholds(NK, E):
    """Either side of the limits up to which the scatter finds a round's same-expert
    lanes through LDS masks (below 2^21 slots, up to 256 experts) rather than one ballot
    per expert-id bit: both forms must give the same unique stable order."""
    rng = np.random.default_rng(NK + E)
    idx = rng.integers(0, E, size=(NK, 1)).astype(np.int32)
    idx[rng.random((NK, 1)) < 0.2] = -1
    w = rng.standard_normal((NK, 1)).astype(np.float32)
    check(idx, w, E)


@pytest.mark.parametrize("N,K", [(32768, 8), (131072, 8)])
def test_slot_count_thresholds_wide_rows(N, K):
    """The same thresholds reached with K = 8 slots per token (token offsets then come
    from slots in the middle of chunks)."""
    rng = np.random.default_rng(N + K)
    E = 64
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    idx[rng.random((N, K)) < 0.2] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    check(idx, w, E)


@pytest.mark.parametrize("NK,E", [(511, 48), (512, 48), (513, 48), (1024, 48), (1025, 48),
                                  (2047, 48), (2048, 48), (2049, 48), (600, 1024),
                                  (2048, 1024)])
def test_one_workgroup_build_limits(NK, E):
    """Either side of the slot counts where the whole build runs in one workgroup (four
    wavefronts up to 512 slots, eight of two rounds up to 1024, eight of four rounds up to
    2048) and where it takes the multi-chunk launches; up to 1024 experts."""
    rng = np.random.default_rng(NK + E)
    idx = rng.integers(0, E, size=(NK, 1)).astype(np.int32)
    idx[rng.random((NK, 1)) < 0.2] = -1
    w = rng.standard_normal((NK, 1)).astype(np.float32)
    check(idx, w, E)


@pytest.mark.parametrize("N,K,E", [(8, 8, 32), (64, 8, 1024), (128, 8, 64), (256, 8, 64),
                                   (257, 8, 64)])
def test_one_workgroup_build_rows(N, K, E):
    """Decode-sized batches with K = 8 slots per token, duplicates and -1 slots, bad ids
    (flagged, treated as -1) and a capacity below P."""
    rng = np.random.default_rng(N * K + E)
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    idx[rng.random((N, K)) < 0.2] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    got = check(idx, w, E)
    P = got["P"]
    if P > 3:
        check(idx, w, E, capacity=P - 3, expect_status=2)
    bad = idx.copy()
    bad[0, 0] = E
    d = dict(N=N, H=128, I=128, E=E, K=K, topk_idx=bad, topk_weights=w,
             x=np.zeros((N, 128), np.uint16), w_up=np.zeros((E, 128, 256), np.uint16),
             w_down=np.zeros((E, 128, 128), np.uint16))
    clean = np.where(bad < E, bad, -1)
    ref = oracle.build_metadata(clean, w, E)
    g = Gpu(d, capacity=max(ref["P"], 1))
    g.build()
    m = g.meta_numpy()
    assert m["status"] == 1
    for k in KEYS:
        r = ref[k][:ref["P"]] if k in PAIR_KEYS else ref[k]
        assert np.array_equal(m[k], r.astype(m[k].dtype)), k


@pytest.mark.parametrize("NK", [5000, (1 << 20) + 3, (1 << 22) + 5])
def test_inputs_with_element_alignment_only(NK):
    """topk_idx and topk_weights starting 4 bytes past a 16-byte boundary (views one
    element into larger buffers): the C ABI asks for element alignment only, so the
    build must give the oracle's metadata bit for bit at each chunk size."""
    import torch

    import token_routing_grouped_amd as moe

    rng = np.random.default_rng(NK)
    E = 40
    idx = rng.integers(0, E, size=(NK, 1)).astype(np.int32)
    idx[rng.random((NK, 1)) < 0.2] = -1
    w = rng.standard_normal((NK, 1)).astype(np.float32)
    print(f"metadata case NK={NK} E={E}, inputs offset by one element", flush=True)
    ref = oracle.build_metadata(idx, w, E)
    buf = torch.empty(NK + 4, dtype=torch.int32, device="cuda")
    ti = buf[1:1 + NK].view(NK, 1)
    ti.copy_(torch.from_numpy(idx))
    assert ti.data_ptr() % 16 == 4
    wbuf = torch.empty(NK + 4, dtype=torch.float32, device="cuda")
    tw = wbuf[1:1 + NK].view(NK, 1)
    tw.copy_(torch.from_numpy(w))
    assert tw.data_ptr() % 16 == 4
    meta = moe.Metadata(NK, 1, E, NK, device="cuda")
    moe.moe_build_metadata(ti, tw, meta)
    torch.cuda.synchronize()
    P = ref["P"]
    assert int(meta.status.item()) == 0
    for k in KEYS:
        got = getattr(meta, k).cpu().numpy()
        if k in PAIR_KEYS:
            got = got[:P]
        assert np.array_equal(got, ref[k].astype(got.dtype)), k
