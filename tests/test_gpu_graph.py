"""The whole path (metadata build, forward, backward) captured in one HIP graph.

The metadata is built on the device from topk_idx without a host round trip (the
pair count never leaves the GPU; kernels size their work from the capacity and
read the true counts on the device), so the three calls capture. The graph is
replayed several times, with eager work, output clobbering and synchronisations
between replays, alternating two routings of the same shape: every replay must
reproduce, bit for bit, the eager result for the routing it was given. The eager
results themselves are checked against the oracle by the other GPU tests; here
one replay is also checked against the oracle directly.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, assert_close, f64, np64

pytestmark = pytest.mark.gpu


def _dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def test_graph_replay_matches_eager():
    import torch
    import token_routing_grouped_amd as moe

    N, H, I, E, K = 700, 256, 384, 8, 4
    cases = [synth.case(N, H, I, E, K, seed=s, p_invalid=0.2) for s in (11, 12)]
    print(f"graph case N={N} H={H} I={I} E={E} K={K}", flush=True)
    cap = N * K
    meta = moe.Metadata(N, K, E, cap, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x = torch.empty(N, H, **bf)
    w_up = torch.empty(E, H, 2 * I, **bf)
    w_down = torch.empty(E, I, H, **bf)
    dout = torch.empty(N, H, **bf)
    idx = torch.empty(N, K, dtype=torch.int32, device="cuda")
    wts = torch.empty(N, K, dtype=torch.float32, device="cuda")
    out = torch.empty(N, H, **bf)
    h = torch.empty(cap, 2 * I, **bf)
    dx = torch.empty(N, H, **bf)
    dw_up = torch.empty(E, H, 2 * I, **bf)
    dw_down = torch.empty(E, I, H, **bf)
    dtw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    ws_m = torch.empty(max(1, moe.moe_build_metadata_workspace(N, K, E)), **u8)
    ws_f = torch.empty(max(1, moe.moe_expert_forward_workspace(meta, H, I)), **u8)
    ws_b = torch.empty(max(1, moe.moe_expert_backward_workspace(meta, H, I)), **u8)

    def load(d):
        x.copy_(_dev_bf16(torch, d["x"]))
        w_up.copy_(_dev_bf16(torch, d["w_up"]))
        w_down.copy_(_dev_bf16(torch, d["w_down"]))
        dout.copy_(_dev_bf16(torch, d["dout"]))
        idx.copy_(torch.from_numpy(d["topk_idx"]))
        wts.copy_(torch.from_numpy(d["topk_weights"]))

    def step():
        moe.moe_build_metadata(idx, wts, meta, workspace=ws_m)
        moe.moe_expert_forward(meta, x, w_up, w_down, out, h_save=h, workspace=ws_f)
        moe.moe_expert_backward(meta, idx, x, w_up, w_down, h, dout, dx, dw_up, dw_down, dtw,
                                workspace=ws_b)

    def clobber():
        for t in (out, h, dx, dw_up, dw_down, dtw, meta.router_scores):
            t.fill_(float("nan"))
        for t in (meta.expert_frequency, meta.expert_frequency_offset, meta.x_gather_idx,
                  meta.s_scatter_idx, meta.s_reverse_scatter_idx,
                  meta.num_activated_expert_per_token_offset, meta.status):
            t.fill_(-7)

    def snapshot(P):
        return dict(
            out=out.clone(), h=h[:P].clone(), dx=dx.clone(), dw_up=dw_up.clone(),
            dw_down=dw_down.clone(), dtw=dtw.clone(),
            expert_frequency=meta.expert_frequency.clone(),
            expert_frequency_offset=meta.expert_frequency_offset.clone(),
            x_gather_idx=meta.x_gather_idx[:P].clone(),
            s_scatter_idx=meta.s_scatter_idx[:P].clone(),
            s_reverse_scatter_idx=meta.s_reverse_scatter_idx[:P].clone(),
            tok_off=meta.num_activated_expert_per_token_offset.clone(),
            router_scores=meta.router_scores[:P].clone(),
            status=meta.status.clone())

    Ps = [int((d["topk_idx"] >= 0).sum()) for d in cases]
    refs = []
    for d, P in zip(cases, Ps):
        load(d)
        clobber()
        step()
        torch.cuda.synchronize()
        refs.append(snapshot(P))
        assert int(refs[-1]["status"].item()) == 0

    # capture on a side stream (warmed up there first)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()

    other = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        c = rep % 2
        print(f"replay {rep} routing {c}", flush=True)
        load(cases[c])
        clobber()
        _ = (other @ other).sum().item()  # unrelated eager work and a host sync
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(Ps[c])
        for k, ref in refs[c].items():
            assert torch.equal(got[k], ref), f"replay {rep}: {k} differs from the eager result"

    # the last replay (routing 1) against the oracle as well
    d = cases[1]
    m = oracle.build_metadata(d["topk_idx"], d["topk_weights"], E)
    assert np.array_equal(meta.x_gather_idx[:Ps[1]].cpu().numpy(), m["x_gather_idx"])
    f = oracle.forward(f64(d["x"]), f64(d["w_up"]), f64(d["w_down"]), m)
    assert_close(np64(out), f["out"], TOL["bf16"], "out")
