"""The allocation-free metadata build (moe_build_metadata_noalloc, for callers that
cannot allocate device memory) against the workspace entry point moe_build_metadata:
bit-identical metadata on two calls in a row, the second smaller than the first (the
library's static scratch then holds the first call's contents), and a build larger
than the scratch refused synchronously."""
import numpy as np
import pytest

import oracle
import synth
from _util import Gpu

pytestmark = pytest.mark.gpu

KEYS = ["expert_frequency", "expert_frequency_offset", "x_gather_idx", "s_scatter_idx",
        "s_reverse_scatter_idx", "num_activated_expert_per_token_offset", "router_scores",
        "status"]


def both_ways(d, capacity=None):
    """(workspace build, allocation-free build) of the same inputs, as numpy dicts."""
    import token_routing_grouped_amd as moe

    ga = Gpu(d, capacity=capacity)
    ga.build()
    gb = Gpu(d, capacity=capacity)
    # poison the outputs so that a skipped write cannot pass
    for t in (gb.meta.expert_frequency, gb.meta.expert_frequency_offset, gb.meta.x_gather_idx,
              gb.meta.s_scatter_idx, gb.meta.s_reverse_scatter_idx,
              gb.meta.num_activated_expert_per_token_offset, gb.meta.status):
        t.fill_(-7)
    gb.meta.router_scores.fill_(float("nan"))
    moe.moe_build_metadata_noalloc(gb.topk_idx, gb.topk_weights, gb.meta)
    ga.torch.cuda.synchronize()
    return ga.meta_numpy(), gb.meta_numpy()


def check_same(a, b, d):
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k
    m = oracle.build_metadata(d["topk_idx"], d["topk_weights"], d["E"])
    for k in KEYS[:-1]:
        assert np.array_equal(b[k], m[k].astype(b[k].dtype)), k


def test_noalloc_matches_workspace_build_twice():
    import token_routing_grouped_amd as moe

    big = synth.make_inputs("qwen3_rank", 0, dout=False)
    big_ws = moe.moe_build_metadata_workspace(big["N"], big["K"], big["E"])
    # 2100 slots: above the 2048 a single workgroup builds without any workspace, so the
    # second call also runs through the scratch array (five chunks, two launches)
    small = synth.case(N=700, H=128, I=128, E=12, K=3, seed=51, p_invalid=0.3)
    small_ws = moe.moe_build_metadata_workspace(small["N"], small["K"], small["E"])
    assert small_ws < big_ws <= moe.MOE_NOALLOC_SCRATCH_BYTES
    assert small["N"] * small["K"] > 2048
    print(f"noalloc call 1: N={big['N']} K={big['K']} E={big['E']} ({big_ws} bytes)", flush=True)
    a, b = both_ways(big)
    check_same(a, b, big)
    print(f"noalloc call 2: N={small['N']} K={small['K']} E={small['E']} ({small_ws} bytes)",
          flush=True)
    a, b = both_ways(small)
    check_same(a, b, small)


def test_noalloc_over_capacity_and_bad_ids():
    # data errors take the same device status path as the workspace build
    d = synth.case(N=300, H=128, I=128, E=6, K=3, seed=52)
    d["topk_idx"][5, 1] = 77
    P = int(((d["topk_idx"] >= 0) & (d["topk_idx"] < 6)).sum())
    print("noalloc: bad id and capacity below P", flush=True)
    a, b = both_ways(d, capacity=P - 9)
    assert a["status"] == b["status"] == 3
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_noalloc_refuses_builds_beyond_the_scratch():
    import torch

    import token_routing_grouped_amd as moe

    # 1024 experts over 2^21 slots need more workspace than the static scratch holds
    N, K, E = 1 << 18, 8, 1024
    assert moe.moe_build_metadata_workspace(N, K, E) > moe.MOE_NOALLOC_SCRATCH_BYTES
    meta = moe.Metadata(N, K, E, 16, device="cuda")
    idx = torch.full((N, K), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    meta.status.fill_(-7)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_build_metadata_noalloc(idx, w, meta)
    assert ei.value.status == moe._binding.MOE_ENOSPC
    torch.cuda.synchronize()
    assert int(meta.status.item()) == -7  # nothing was enqueued


def test_noalloc_build_in_a_hip_graph():
    """The allocation-free build is what graph capture calls for: captured once (after a
    first eager call has looked up the scratch address), replayed with two routings of one
    shape loaded into the same input buffers, eager work and synchronisations between the
    replays; every replay must equal, bit for bit, the workspace build of that routing."""
    import torch

    import token_routing_grouped_amd as moe

    N, K, E = 3000, 8, 32
    cases = [synth.make_inputs(dict(N=N, H=128, I=128, E=E, K=K, routing="ep_share",
                                    global_experts=256), seed=s, dout=False)
             for s in (3, 4)]
    print(f"noalloc graph case N={N} K={K} E={E}", flush=True)
    cap = N * K
    idx = torch.empty(N, K, dtype=torch.int32, device="cuda")
    wts = torch.empty(N, K, dtype=torch.float32, device="cuda")
    meta = moe.Metadata(N, K, E, cap, device="cuda")
    refs = []
    for d in cases:
        r = moe.Metadata(N, K, E, cap, device="cuda")
        moe.moe_build_metadata(torch.from_numpy(d["topk_idx"]).cuda(),
                               torch.from_numpy(d["topk_weights"]).cuda(), r)
        torch.cuda.synchronize()
        P = int(r.expert_frequency_offset[-1].item())
        refs.append({k: getattr(r, k).cpu().numpy()[:P] if k in (
            "x_gather_idx", "s_scatter_idx", "s_reverse_scatter_idx", "router_scores")
            else getattr(r, k).cpu().numpy() for k in KEYS[:-1]})
    idx.copy_(torch.from_numpy(cases[0]["topk_idx"]))
    wts.copy_(torch.from_numpy(cases[0]["topk_weights"]))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        moe.moe_build_metadata_noalloc(idx, wts, meta, stream=stream)  # eager: address lookup
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        moe.moe_build_metadata_noalloc(idx, wts, meta, stream=stream)
    torch.cuda.synchronize()
    for rep in range(6):
        c = rep % 2
        idx.copy_(torch.from_numpy(cases[c]["topk_idx"]))
        wts.copy_(torch.from_numpy(cases[c]["topk_weights"]))
        meta.x_gather_idx.fill_(-5)  # clobber between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(meta.status.item()) == 0
        P = int(meta.expert_frequency_offset[-1].item())
        for k, ref in refs[c].items():
            got = getattr(meta, k).cpu().numpy()
            if k in ("x_gather_idx", "s_scatter_idx", "s_reverse_scatter_idx", "router_scores"):
                got = got[:P]
            assert np.array_equal(got, ref), (rep, k)



def launches_of(kernel, fn):
    """How many launches of `kernel` fn enqueues (counted by the timing hook)."""
    import torch

    import token_routing_grouped_amd as moe

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    moe.moe_time_kernel(kernel, ev)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        n = moe.moe_time_kernel(kernel, None)
    return n


def test_noalloc_at_the_two_launch_limits():
    """The allocation-free build through the scratch array at both limits of the
    two-launch form (256 chunks of 512 slots; 34 experts), with an invalid expert id and
    capacity below P, and just past each limit (257 chunks; 35 experts), where the column
    scan is a launch of its own: every call bit-identical to the workspace build, and the
    scan launched exactly where the limits say."""
    import torch

    import token_routing_grouped_amd as moe

    cases = [
        ("256 chunks, 32 experts", dict(N=16384, H=128, I=128, E=32, K=8, seed=71), None, 0),
        ("34 experts", dict(N=5000, H=128, I=128, E=34, K=6, seed=72, p_invalid=0.2), None, 0),
        ("257 chunks", dict(N=16385, H=128, I=128, E=32, K=8, seed=73), None, 1),
        ("35 experts", dict(N=5000, H=128, I=128, E=35, K=6, seed=74), None, 1),
        ("bad id, capacity below P", dict(N=1000, H=128, I=128, E=20, K=3, seed=75), "err", 0),
    ]
    for name, kw, kind, scans in cases:
        d = synth.case(**kw)
        cap = None
        if kind == "err":
            d["topk_idx"][17, 2] = 40
            cap = int(((d["topk_idx"] >= 0) & (d["topk_idx"] < kw["E"])).sum()) - 11
        print(f"noalloc case: {name} N={kw['N']} K={kw['K']} E={kw['E']}", flush=True)
        a, b = both_ways(d, capacity=cap)
        if kind == "err":
            assert a["status"] == b["status"] == 3
            for k in KEYS:
                assert np.array_equal(a[k], b[k]), k
        else:
            assert b["status"] == 0
            check_same(a, b, d)
        g = Gpu(d, capacity=cap)
        torch.cuda.synchronize()
        n = launches_of("meta_scan", lambda: moe.moe_build_metadata_noalloc(
            g.topk_idx, g.topk_weights, g.meta))
        assert n == scans, name
