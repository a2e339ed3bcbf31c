"""GPU router (moe_route: top-K, weights, aux loss, and the metadata in the same pass)
against the oracle, through the C ABI.

Selection and every metadata array are compared bit for bit: the top-K choice is
decided on the given fp32 (or bf16) logit values on both sides. The weights are fp32
softmax values in [0,1] against the fp64 oracle: max abs error <= 2e-6 (a few fp32
ulps of exp and one division); the aux loss (a sum of N*E fp32 terms in a fixed order)
within 1e-5 relative. Shapes cover chunks of the slot layout that split a token's slots
(K not dividing the chunk), E up to 1024 and K up to 64, ties, both modes and the
renormalised one, bf16 logits, and N = 0.
"""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL, assert_close, f64, np64

pytestmark = pytest.mark.gpu

W_TOL = 2e-6
AUX_RTOL = 1e-5


def run_route(lg_np, K, mode, renorm, dtype="fp32", capacity=None):
    import torch
    import token_routing_grouped_amd as moe

    N, E = lg_np.shape
    print(f"route N={N} E={E} K={K} mode={mode} renorm={renorm} dtype={dtype}", flush=True)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(lg_np)
        lg = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        ref_in = bits
    else:
        lg = torch.from_numpy(np.ascontiguousarray(lg_np)).cuda()
        ref_in = lg_np
    meta = moe.Metadata(N, K, E, N * K if capacity is None else capacity, device="cuda")
    idx, w, aux = moe.moe_route(lg, meta, mode=mode, renormalize=renorm)
    torch.cuda.synchronize()
    ref = oracle.route(ref_in, K, mode, renormalize=renorm)
    return meta, idx.cpu().numpy(), w.cpu().numpy(), float(aux.cpu().numpy()[0]), ref


def check(meta, idx, w, aux, ref):
    assert np.array_equal(idx, ref["topk_idx"])
    err = np.max(np.abs(w.astype(np.float64) - ref["topk_weights"])) if w.size else 0.0
    assert err <= W_TOL, f"weights max err {err:.3e}"
    assert aux == pytest.approx(ref["aux"], rel=AUX_RTOL, abs=1e-12)
    # the metadata built in the same pass equals the oracle's metadata of these outputs
    m = oracle.build_metadata(idx, w, meta.E)
    c = lambda t: t.cpu().numpy()
    P = m["P"]
    assert np.array_equal(c(meta.expert_frequency), m["expert_frequency"])
    assert np.array_equal(c(meta.expert_frequency_offset), m["expert_frequency_offset"])
    assert np.array_equal(c(meta.num_activated_expert_per_token_offset),
                          m["num_activated_expert_per_token_offset"])
    assert np.array_equal(c(meta.x_gather_idx)[:P], m["x_gather_idx"])
    assert np.array_equal(c(meta.s_scatter_idx)[:P], m["s_scatter_idx"])
    assert np.array_equal(c(meta.s_reverse_scatter_idx)[:P], m["s_reverse_scatter_idx"])
    assert np.array_equal(c(meta.router_scores)[:P], m["router_scores"])
    assert int(c(meta.status)[0]) == 0


@pytest.mark.parametrize("mode,renorm", [(0, False), (1, False), (1, True)])
@pytest.mark.parametrize("N,E,K", [(1000, 8, 2), (777, 64, 6), (513, 128, 8), (300, 256, 8),
                                   (64, 1000, 16), (5, 1024, 64)])
def test_route_fp32(N, E, K, mode, renorm):
    lg = synth.router_logits(N, E, seed=N + E + K)
    check(*run_route(lg, K, mode, renorm))


@pytest.mark.parametrize("mode", [0, 1])
def test_route_bf16_logits_with_ties(mode):
    lg = synth.router_logits(900, 64, seed=2, ties=True)
    check(*run_route(lg, 8, mode, False, dtype="bf16"))


def test_route_k_equals_e_and_k1():
    lg = synth.router_logits(200, 16, seed=4)
    check(*run_route(lg, 16, 0, False))
    check(*run_route(lg, 1, 1, False))


def test_route_empty():
    lg = np.zeros((0, 32), np.float32)
    meta, idx, w, aux, ref = run_route(lg, 4, 0, False)
    assert aux == 0.0
    assert np.all(meta.expert_frequency_offset.cpu().numpy() == 0)
    assert np.all(meta.num_activated_expert_per_token_offset.cpu().numpy() == 0)


def test_route_then_forward():
    """moe_route's outputs feed the expert forward directly; the result equals the
    oracle forward on the oracle router's choice."""
    import torch
    import token_routing_grouped_amd as moe

    N, H, I, E, K = 400, 256, 128, 16, 4
    lg = synth.router_logits(N, E, seed=12)
    d = synth.case(N, H, I, E, K, seed=12, topk_idx=np.zeros((N, K), np.int32))
    meta, idx, w, aux, ref = run_route(lg, K, 1, True)
    check(meta, idx, w, aux, ref)
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(
        torch.bfloat16).cuda()
    out = torch.empty(N, H, dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_forward(meta, bf(d["x"]), bf(d["w_up"]), bf(d["w_down"]), out)
    m = oracle.build_metadata(ref["topk_idx"], ref["topk_weights"].astype(np.float32), E)
    f = oracle.forward(f64(d["x"]), f64(d["w_up"]), f64(d["w_down"]), m)
    assert_close(np64(out), f["out"], TOL["bf16"], "out")


@pytest.mark.parametrize("N,E", [(300000, 64), (600000, 32)])
def test_route_long_columns(N, E):
    """Over 2048 metadata chunks (of 1024 slots at 2.4M slots, of 2048 at 4.8M): the
    counts and the aux loss's probability columns are reduced in two passes."""
    lg = synth.router_logits(N, E, seed=21)
    check(*run_route(lg, 8, 1, False))


@pytest.mark.parametrize("N,K", [(32768, 8), (131072, 8), (262143, 4), (524288, 8)])
def test_route_slot_count_thresholds(N, K):
    """Router at the slot counts where the metadata chunks and the scatter's write-out
    change (2^18, 2^20 and 2^22 slots), and a ragged last chunk."""
    lg = synth.router_logits(N, 32, seed=N + K)
    check(*run_route(lg, K, 1, True))
