"""CPU pins of the oracle's router (the Hysen Labs page on Dao-AILab/sonic-moe,
section "Three routing strategies, selected on the command line").

- selection: the K largest logits, largest first, equal logits to the lower expert
  id, checked against numpy's stable argsort of the negated logits;
- softmax over the top-K: the weights are numpy's softmax of the selected logits;
- top-K of the softmax: the weights are numpy's softmax over all E at the selected
  experts; renormalised, they equal the softmax over the top-K (the two orders agree
  once renormalised);
- K = E: softmax over the top-K is the full softmax;
- aux loss (E * sum_e f_e * P_e): hand-computed closed forms.
"""
import numpy as np
import pytest

import oracle
import synth


def np_softmax(a, axis=-1):
    m = np.max(a, axis=axis, keepdims=True)
    z = np.exp(a - m)
    return z / z.sum(axis=axis, keepdims=True)


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("N,E,K", [(50, 8, 2), (40, 64, 6), (9, 300, 17)])
def test_selection_and_weights(N, E, K, ties):
    lg = synth.router_logits(N, E, seed=3, ties=ties).astype(np.float64)
    want_idx = np.argsort(-lg, axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(lg, want_idx, axis=1)
    r0 = oracle.route(lg, K, 0)
    assert np.array_equal(r0["topk_idx"], want_idx)
    assert np.allclose(r0["topk_weights"], np_softmax(sel), rtol=1e-13, atol=1e-15)
    r1 = oracle.route(lg, K, 1)
    assert np.array_equal(r1["topk_idx"], want_idx)
    full = np_softmax(lg)
    assert np.allclose(r1["topk_weights"], np.take_along_axis(full, want_idx, axis=1),
                       rtol=1e-13, atol=1e-15)
    r1n = oracle.route(lg, K, 1, renormalize=True)
    assert np.allclose(r1n["topk_weights"], r0["topk_weights"], rtol=1e-13, atol=1e-15)
    assert np.allclose(r1n["topk_weights"].sum(axis=1), 1.0, rtol=1e-13)


def test_k_equals_e_is_full_softmax():
    lg = synth.router_logits(20, 12, seed=5).astype(np.float64)
    r = oracle.route(lg, 12, 0)
    full = np_softmax(lg)
    assert np.allclose(r["topk_weights"], np.take_along_axis(full, r["topk_idx"], axis=1),
                       rtol=1e-13)
    assert np.array_equal(np.sort(r["topk_idx"], axis=1), np.tile(np.arange(12), (20, 1)))


def test_aux_closed_forms():
    # two tokens, two experts, K=1, each token on its own expert: f = P = (1/2, 1/2)
    # -> aux = 2 * (1/4 + 1/4) = 1
    assert oracle.route(np.array([[1.0, 0.0], [0.0, 1.0]]), 1, 1)["aux"] == pytest.approx(1.0, abs=1e-15)
    # both tokens on expert 0: f = (1, 0), P_0 = (sigmoid(2) + sigmoid(1)) / 2
    # -> aux = 2 * P_0 = sigmoid(2) + sigmoid(1)
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    got = oracle.route(np.array([[2.0, 0.0], [1.0, 0.0]]), 1, 0)["aux"]
    assert got == pytest.approx(sig(2.0) + sig(1.0), rel=1e-14)
    # all logits equal: every token picks experts 0..K-1 (lower id on ties), P_e = 1/E
    # -> aux = E * K * (1/K) * (1/E) = 1
    r = oracle.route(np.zeros((7, 10)), 3, 1)
    assert np.all(r["topk_idx"] == np.arange(3))
    assert r["aux"] == pytest.approx(1.0, rel=1e-14)
    # the aux loss does not depend on the weighting mode
    lg = synth.router_logits(30, 16, seed=8).astype(np.float64)
    assert oracle.route(lg, 4, 0)["aux"] == pytest.approx(oracle.route(lg, 4, 1)["aux"], rel=1e-15)


def test_typed_inputs_take_the_same_decisions():
    lg32 = synth.router_logits(60, 32, seed=9, ties=True)
    bits = synth.f32_to_bf16_bits(lg32)
    r_b = oracle.route(bits, 5, 0)
    r_f = oracle.route(synth.bf16_bits_to_f32(bits), 5, 0)
    assert np.array_equal(r_b["topk_idx"], r_f["topk_idx"])
    assert np.array_equal(r_b["topk_weights"], r_f["topk_weights"])
