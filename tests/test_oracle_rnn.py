"""Pins for the oracle's RNN head (CPU only).

The pages describe the RNN head only in words (a gated update of an in-block
recurrent state over the concatenated history state, previous-token embedding
and backbone hidden state); the oracle follows one stated reading.  These
tests pin that reading against things that do not depend on the oracle's
code: its reduction to the (separately pinned) Markov head when the gate is
saturated open, a frozen state when the gate is shut, the closed form of the
recurrence at a half-open gate, a known tanh offset of the candidate, which
input block drives a gate, and the two-rounding bf16 conversion of the state.
"""
import dataclasses

import numpy as np
import pytest

from oracle import dspark_oracle as O
from draft_head_step_amd.inputs import (CONFIGS, SAMPLE, Config, f32_to_bf16_bits, make_rnn_head,
                                         make_workload)


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _head(r, d, gate_bias, cand_bias=0.0, gate_w=None, seed=0):
    """U with an optional gate block and a zero candidate block; b = [gate; cand]."""
    U = np.zeros((2 * r, 2 * r + d), np.float32)
    if gate_w is not None:
        U[:r] = gate_w
    b = np.concatenate([np.full(r, gate_bias), np.full(r, cand_bias)]).astype(np.float32)
    return _bf16(U), b


@pytest.mark.parametrize("mode", [O.GREEDY, O.SAMPLE])
def test_saturated_gate_reduces_to_the_markov_head(mode):
    # g = sigmoid(G u + 100) = 1 whatever G u is (|G u| < 10 here); C = 0 and
    # b_c = 0 make the candidate the embedding row: s_k = W1[x_{k-1}].
    cfg = CONFIGS["tiny"]
    if mode == O.SAMPLE:
        cfg = dataclasses.replace(cfg, mode=SAMPLE, temperature=0.8)
    wl = make_workload(cfg, w_std=0.3)
    r, d = wl["r"], wl["d"]
    rng = np.random.default_rng(1)
    U, b = _head(r, d, 100.0, gate_w=rng.uniform(-0.02, 0.02, size=(r, 2 * r + d)))
    rn = O.rnn_draft(wl["W1"], wl["W2"], U, b, wl["base"], wl["h"], wl["anchors"], mode,
                     wl["temperature"], wl["uniforms"], keep_state=True)
    mk = O.markov_draft(wl["W1"], wl["W2"], wl["base"], wl["anchors"], mode, wl["temperature"],
                        wl["uniforms"])
    assert np.array_equal(rn["tokens"], mk["tokens"])
    np.testing.assert_allclose(rn["margin"], mk["margin"], rtol=0, atol=1e-12)
    prev = np.concatenate([wl["anchors"][:, None], mk["tokens"][:, :-1]], axis=1)
    np.testing.assert_allclose(rn["states"], O.bf16_to_f64(wl["W1"][prev]), rtol=0, atol=1e-30)


def test_shut_gate_freezes_the_zero_state():
    # g = sigmoid(-100) ~ 0: the state stays s_0 = 0, so no bias is added and the
    # draft is the argmax of the base logits (checked with plain Python max).
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    U, b = _head(wl["r"], wl["d"], -100.0)
    rn = O.rnn_draft(wl["W1"], wl["W2"], U, b, wl["base"], wl["h"], wl["anchors"], keep_state=True)
    assert np.abs(rn["states"]).max() < 1e-40
    R, g, V = wl["base"].shape
    for m in range(R):
        for k in range(g):
            row = [float(v) for v in wl["base"][m, k]]
            assert rn["tokens"][m, k] == max(range(V), key=lambda v: (row[v], -v))


def test_half_open_gate_is_an_exponential_average_of_the_embeddings():
    # U = 0, b = 0: g = 1/2 and tanh(0) = 0, so s_k = (e_k + s_{k-1}) / 2, i.e.
    # s_k = sum_j 2^-(k-j+1) e_j.  Embedding entries in {-2..2} keep every state
    # exactly representable in bf16.
    rng = np.random.default_rng(4)
    V, r, d, R, g = 40, 16, 8, 3, 4
    W1 = _bf16(rng.integers(-2, 3, size=(V, r)))
    W2 = _bf16(rng.standard_normal((V, r)) * 0.5)
    base = rng.standard_normal((R, g, V)).astype(np.float32)
    h = _bf16(rng.standard_normal((R, g, d)))
    anchors = np.array([1, 17, 39], np.int32)
    U, b = _head(r, d, 0.0)
    rn = O.rnn_draft(W1, W2, U, b, base, h, anchors, keep_state=True)
    prev = np.concatenate([anchors[:, None], rn["tokens"][:, :-1]], axis=1)
    E = O.bf16_to_f64(W1[prev])                                  # [R, g, r]
    for k in range(g):
        want = sum(E[:, j, :] * 2.0 ** -(k - j + 1) for j in range(k + 1))
        assert np.array_equal(rn["states"][:, k, :], want)
        bias = want @ O.bf16_to_f64(W2).T                        # exact states: no rounding
        assert np.array_equal(rn["tokens"][:, k], np.argmax(base[:, k] + bias, axis=1))


def test_candidate_offset_through_tanh():
    # Open gate, C = 0, b_c = atanh(1/2): s_k = e_k + 1/2, so the bias is the
    # Markov bias plus half the column sums of W2.
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    rng = np.random.default_rng(5)
    W1 = _bf16(rng.integers(-3, 4, size=wl["W1"].shape))
    U, b = _head(wl["r"], wl["d"], 100.0, cand_bias=np.arctanh(0.5))
    rn = O.rnn_draft(W1, wl["W2"], U, b, wl["base"], wl["h"], wl["anchors"], keep_state=True)
    prev = np.concatenate([wl["anchors"][:, None], rn["tokens"][:, :-1]], axis=1)
    # (b_c is fp32, so tanh(b_c) is 1/2 to about 1e-8)
    np.testing.assert_allclose(rn["states"], O.bf16_to_f64(W1[prev]) + 0.5, rtol=0, atol=1e-7)
    col = O.w2_matrix(wl["W2"]).sum(axis=0)
    for k in range(wl["gamma"]):
        bias = O.markov_bias(W1, wl["W2"], prev[:, k]) + 0.5 * col
        assert np.array_equal(rn["tokens"][:, k], np.argmax(wl["base"][:, k] + bias, axis=1))


@pytest.mark.parametrize("block", ["s", "e", "h"])
def test_each_input_block_drives_the_gate_it_should(block):
    # Gate unit n gets weight 1024 on one input of one block (the state's unit n,
    # the embedding's unit n, or hidden unit n), every other gate weight 0 and a
    # zero candidate correction: unit n copies e_n where that input is positive
    # and keeps its state where it is negative (g saturates at 1 or 0).
    rng = np.random.default_rng(6)
    V, r, d, R, g = 32, 8, 8, 4, 5
    W1 = _bf16(rng.choice([-1.0, -0.5, 0.5, 1.0], size=(V, r)))
    W2 = _bf16(rng.standard_normal((V, r)))
    base = rng.standard_normal((R, g, V)).astype(np.float32)
    h = _bf16(rng.choice([-1.0, 1.0], size=(R, g, d)))
    anchors = rng.integers(0, V, size=R).astype(np.int32)
    G = np.zeros((r, 2 * r + d), np.float32)
    off = {"s": 0, "e": r, "h": 2 * r}[block]
    for n in range(r):
        G[n, off + n] = 1024.0     # |input| >= 1/4: the gate saturates to within e^-256
    U, b = _head(r, d, 0.0, gate_w=G)
    rn = O.rnn_draft(W1, W2, U, b, base, h, anchors, keep_state=True)
    prev = np.concatenate([anchors[:, None], rn["tokens"][:, :-1]], axis=1)
    E = O.bf16_to_f64(W1[prev])
    H = O.bf16_to_f64(h)
    s = np.zeros((R, r))
    for k in range(g):
        drive = {"s": s, "e": E[:, k], "h": H[:, k, :r]}[block]
        s = np.where(drive > 0, E[:, k], s)          # drive is never 0 here (except s at k = 0)
        if block == "s" and k == 0:
            s = np.zeros((R, r)) * 0.5 + 0.5 * E[:, 0]   # sigmoid(0) = 1/2 on the zero state
        np.testing.assert_allclose(rn["states"][:, k], s, rtol=0, atol=1e-30)


def test_bf16_round_is_two_roundings_to_nearest_even():
    # fp64 -> fp32 -> bf16, each to nearest even (so 1 + 2^-8 + 2^-30 first becomes
    # the fp32 1 + 2^-8, a bf16 tie, and then rounds down to 1).
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -2.5,
                  3.0 * 2 ** -130, np.inf, -np.inf])
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, np.inf, -np.inf])
    got = O.bf16_round(x)
    assert np.array_equal(got[:5], want[:5]) and np.isinf(got[6:]).all()
    assert abs(got[5]) < 2 ** -126
    assert np.isnan(O.bf16_round(np.array([np.nan])))[0]


def test_synthetic_rnn_head_keeps_gates_in_their_working_range():
    # The seeded head's pre-activations are of order one on the workload's inputs
    # (neither saturated nor constant), so the recurrence is exercised.
    cfg = Config("edge", R=8, gamma=3, V=3000, r=64, d=256, w_std=0.05, seed=9)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    rn = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                     keep_state=True)
    st = rn["states"]
    assert np.all(np.isfinite(st)) and 0.05 < np.abs(st).mean() < 2.0


def test_the_state_enters_both_products_rounded_to_bf16():
    # A hand-worked three-step chain (r = 1, d = 1, V = 2, one request) where the
    # bf16 rounding of the state decides both a token and a gate:
    #   step 1: s_0 = 0, pre_g = 0 -> g = 1/2, e_1 = W1[0] = 2^-7, s_1 = 2^-8;
    #           z = [0, 1] + s_1 * [1, 0] -> token 1;
    #   step 2: pre_g = 2^13 * bf16(s_1) - 2^13 * h_2 = 0 (h_2 = 2^-8) -> g = 1/2,
    #           e_2 = W1[1] = 2, s_2 = 1 + 2^-9, whose bf16 value is 1 (a tie, to
    #           even); z = [bf16(s_2), 1 + 2^-10] -> token 1 (the unrounded state
    #           would pick token 0);
    #   step 3: pre_g = 2^13 * bf16(s_2) - 2^13 * h_3 = 0 (h_3 = 1) -> g = 1/2
    #           (unrounded it would be 16: g ~ 1), s_3 = (2 + s_2) / 2 = 1.5 + 2^-10.
    W1 = _bf16([[2.0 ** -7], [2.0]])
    W2 = _bf16([[1.0], [0.0]])                       # stored [V, r]: W2(0, v)
    U = _bf16([[2.0 ** 13, 0.0, -(2.0 ** 13)],       # gate: s, e, h
               [0.0, 0.0, 0.0]])                     # candidate correction: none
    b = np.zeros(2, np.float32)
    base = np.array([[[0.0, 1.0], [0.0, 1.0 + 2.0 ** -10], [0.0, 0.0]]], np.float32)
    h = _bf16([[[0.0], [2.0 ** -8], [1.0]]])
    rn = O.rnn_draft(W1, W2, U, b, base, h, np.array([0], np.int32), keep_state=True)
    assert rn["tokens"][0, 0] == 1 and rn["tokens"][0, 1] == 1
    assert rn["states"][0, 0, 0] == 2.0 ** -8
    assert rn["states"][0, 1, 0] == 1.0 + 2.0 ** -9
    assert rn["states"][0, 2, 0] == 1.5 + 2.0 ** -10
