"""Pins for the oracle's confidence head, STS temperatures and prefix survival (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dspark_oracle as O
from draft_head_step_amd.inputs import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _setup(R=3, g=4, d=6, V=10, r=10, seed=0):
    rng = np.random.default_rng(seed)
    h = _bf16(rng.standard_normal((R, g, d)))
    W1 = _bf16(rng.standard_normal((V, r)))
    anchors = rng.integers(0, V, size=R).astype(np.int32)
    tokens = rng.integers(0, V, size=(R, g)).astype(np.int32)
    return h, W1, anchors, tokens


def test_zero_weights_give_one_half_exactly():
    h, W1, anchors, tokens = _setup()
    c = O.confidence(h, W1, anchors, tokens, np.zeros(6 + 10, np.float32))
    assert c.dtype == np.float32 and np.all(c == np.float32(0.5))


def test_hand_values_and_sts_temperature():
    # h = e_0, w_h = [ln 3, 0...], W1 rows zero: s = ln 3, sigmoid(ln 3) = 3/4;
    # with STS temperature 2: sigmoid(ln 3 / 2) = sqrt(3) / (sqrt(3) + 1).
    R, g, d, V, r = 1, 2, 4, 5, 4
    h = np.zeros((R, g, d), np.float32)
    h[0, :, 0] = 1.0
    W1 = np.zeros((V, r), np.uint16)
    w = np.zeros(d + r, np.float32)
    w[0] = np.log(3.0)
    c = O.confidence(_bf16(h), W1, np.array([0], np.int32), np.zeros((R, g), np.int32), w,
                     sts_temp=np.array([1.0, 2.0], np.float32))
    # w[0] is fp32(ln 3), so compare with the exact sigmoid of that value.
    s = float(np.float32(np.log(3.0)))
    assert c[0, 0] == np.float32(1.0 / (1.0 + np.exp(-s)))
    assert abs(float(c[0, 0]) - 0.75) < 1e-7
    assert abs(float(c[0, 1]) - np.sqrt(3.0) / (np.sqrt(3.0) + 1.0)) < 1e-7


def test_embedding_part_uses_previous_token():
    # h = 0 and W1 one-hot (V = r): s_k = w_e[x_{k-1}] with x_0 = anchor.
    R, g, d, V = 2, 3, 4, 8
    h = np.zeros((R, g, d), np.uint16)
    W1 = _bf16(np.eye(V, dtype=np.float32))
    w = np.zeros(d + V, np.float32)
    w[d:] = np.linspace(-2, 2, V, dtype=np.float32)
    anchors = np.array([3, 6], np.int32)
    tokens = np.array([[1, 7, 2], [0, 5, 4]], np.int32)
    s = O.confidence_logits(h, W1, anchors, tokens, w)
    for m in range(R):
        prevs = [anchors[m]] + list(tokens[m, :-1])
        assert list(s[m]) == [float(w[d + p]) for p in prevs]


def test_hidden_part_is_dot_with_w_h():
    R, g, d, V, r = 2, 2, 5, 3, 3
    rng = np.random.default_rng(4)
    hf = rng.integers(-3, 4, size=(R, g, d)).astype(np.float32)
    w = np.zeros(d + r, np.float32)
    w[:d] = rng.integers(-2, 3, size=d)
    s = O.confidence_logits(_bf16(hf), np.zeros((V, r), np.uint16), np.zeros(R, np.int32),
                            np.zeros((R, g), np.int32), w)
    for m in range(R):
        for k in range(g):
            assert s[m, k] == sum(float(hf[m, k, i]) * float(w[i]) for i in range(d))


def test_sigmoid_symmetry_and_large_temperature():
    h, W1, anchors, tokens = _setup(seed=2)
    w = np.random.default_rng(1).standard_normal(16).astype(np.float32)
    c = O.confidence(h, W1, anchors, tokens, w)
    cneg = O.confidence(h, W1, anchors, tokens, -w)
    assert np.all(np.abs(c.astype(np.float64) + cneg - 1.0) < 2e-7)
    chot = O.confidence(h, W1, anchors, tokens, w, sts_temp=np.full(4, 1e9, np.float32))
    assert np.all(np.abs(chot - 0.5) < 1e-8)


def test_saturation_stays_in_closed_unit_interval():
    h, W1, anchors, tokens = _setup(seed=3)
    w = np.full(16, 1e6, np.float32)
    c = O.confidence(h, W1, anchors, tokens, w)
    assert np.all((c >= 0) & (c <= 1)) and np.all(np.isin(c, [0.0, 1.0]))


# --- survival -------------------------------------------------------------

def test_survival_of_one_half_is_powers_of_two():
    a = O.survival(np.full((3, 7), 0.5, np.float32))
    assert np.array_equal(a, np.broadcast_to(np.float32(2.0) ** -np.arange(1, 8, dtype=np.float32), (3, 7)))


def test_survival_invariants_random():
    rng = np.random.default_rng(8)
    c = rng.uniform(0, 1, size=(200, 9)).astype(np.float32)
    c[::7, 3] = 1.0
    c[::11, 5] = 0.0
    a = O.survival(c)
    assert np.array_equal(a[:, 0], c[:, 0])
    assert np.all(a[:, 1:] <= a[:, :-1]) and np.all(a >= 0) and np.all(a <= 1)


def test_survival_fixture_from_dspark_acceptance_row():
    # Inputs: the per-position conditional acceptance of DSpark printed in the
    # pages' Figure 2 table; expectation: the exact product, to within the
    # rounding of j sequential fp32 multiplications.
    with open(os.path.join(GOLDEN, "dspark_fig2_survival.json")) as f:
        fx = json.load(f)
    c = np.array([fx["conf"]], np.float32)
    a = O.survival(c)
    exact = Fraction(1)
    for j, cj in enumerate(c[0]):
        exact *= Fraction(float(cj))
        rel = abs(Fraction(float(a[0, j])) - exact) / exact
        assert rel <= (j + 1) * Fraction(1, 1 << 24)
        assert abs(float(a[0, j]) - fx["expected_survival"][j]) < 1e-6
