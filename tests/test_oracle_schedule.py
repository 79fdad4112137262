"""Pins for the oracle's hardware-aware prefix scheduler (CPU only).

The scheduler maximises Theta = tau * SPS(B) over every budget B, with
B = sum_r (1 + l_r) and tau = sum_r (1 + sum_{j<=l_r} a_{r,j}).  It is pinned by
exhaustive enumeration of every per-request length vector in exact rational
arithmetic (no sort involved), by closed forms for special SPS curves, by the
threshold / prefix-closure invariants and by the Figure 1 outcome.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dspark_oracle as O
from draft_head_step_amd.inputs import sps_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(a, sps):
    """Enumerate every l in {0..gamma}^R; exact best tau per B, then exact argmax of Theta."""
    R, g = a.shape
    af = [[Fraction(float(a[r, j])) for j in range(g)] for r in range(R)]
    pref = [[sum(af[r][:l], Fraction(0)) for l in range(g + 1)] for r in range(R)]
    best = {}
    for ls in itertools.product(range(g + 1), repeat=R):
        B = sum(1 + l for l in ls)
        tau = sum(1 + pref[r][l] for r, l in enumerate(ls))
        if B not in best or tau > best[B][0]:
            best[B] = (tau, ls)
    theta = {B: best[B][0] * Fraction(float(sps[B - 1])) for B in best}
    top = max(theta.values())
    B_star = min(B for B in theta if theta[B] == top)
    return B_star, best


def _rand_surv(rng, R, g):
    return O.survival(rng.uniform(0.05, 1.0, size=(R, g)).astype(np.float32))


@pytest.mark.parametrize("R,g,seed", [(1, 4, 0), (2, 3, 1), (3, 3, 2), (4, 4, 3), (5, 5, 4), (3, 5, 5)])
def test_matches_exhaustive_enumeration(R, g, seed):
    rng = np.random.default_rng(seed)
    a = _rand_surv(rng, R, g)
    sps = np.sort(rng.uniform(0.1, 1.0, size=R * (1 + g) + 3))[::-1].astype(np.float32)
    B_star, best = brute_force(a, sps)
    got = O.schedule(a, sps)
    assert got["B_star"] == B_star
    # the chosen lengths reach the best tau of that budget
    tau_best, _ = best[B_star]
    tau_got = sum(1 + sum(Fraction(float(a[r, j])) for j in range(got["lengths"][r])) for r in range(R))
    assert tau_got == tau_best
    assert int(got["lengths"].sum()) + R == B_star


@pytest.mark.parametrize("R,g,seed", [(2, 4, 10), (4, 3, 11), (5, 4, 12)])
def test_best_tau_per_budget_is_R_plus_top_survivals(R, g, seed):
    # Greedy-optimality invariant: max tau at budget B = R + sum of the top (B - R) survivals.
    rng = np.random.default_rng(seed)
    a = _rand_surv(rng, R, g)
    sps = np.ones(R * (1 + g), np.float32)
    _, best = brute_force(a, sps)
    desc = sorted((Fraction(float(v)) for v in a.reshape(-1)), reverse=True)
    for B, (tau, _) in best.items():
        assert tau == R + sum(desc[:B - R], Fraction(0))


def test_candidate_order_is_stable_descending():
    rng = np.random.default_rng(21)
    a = O.survival(rng.choice([1.0, 0.75, 0.5], size=(40, 5)).astype(np.float32))
    order = O.candidate_order(a)
    flat = a.reshape(-1)
    want = sorted(range(flat.size), key=lambda i: (-float(flat[i]), i))
    assert list(order) == want


def test_constant_sps_takes_every_candidate():
    rng = np.random.default_rng(2)
    a = _rand_surv(rng, 30, 6)
    got = O.schedule(a, np.ones(30 * 7, np.float32))
    assert got["m_star"] == 180 and np.all(got["lengths"] == 6)


def test_reciprocal_sps_takes_nothing():
    # SPS = 1/B: Theta_0 = R * fl(1/R) ~ 1 while every extension has Theta < 1.
    rng = np.random.default_rng(3)
    a = O.survival(rng.uniform(0.05, 0.99, size=(9, 4)).astype(np.float32))
    B = np.arange(1, 9 * 5 + 1)
    got = O.schedule(a, (1.0 / B).astype(np.float32))
    assert got["m_star"] == 0 and np.all(got["lengths"] == 0)


@pytest.mark.parametrize("K", [7, 20, 33])
def test_step_sps_is_top_k(K):
    # SPS = 1 for B <= K else 0: the schedule is the top (K - R) candidates.
    rng = np.random.default_rng(K)
    R, g = 6, 5
    a = _rand_surv(rng, R, g)
    sps = (np.arange(1, R * (1 + g) + 1) <= K).astype(np.float32)
    got = O.schedule(a, sps)
    assert got["B_star"] == K
    order = sorted(range(R * g), key=lambda i: (-float(a.reshape(-1)[i]), i))
    want = np.bincount(np.array(order[:K - R], dtype=np.int64) // g, minlength=R)
    assert np.array_equal(got["lengths"], want)


def test_selection_is_threshold_set_and_prefix_closed():
    rng = np.random.default_rng(4)
    R, g = 300, 7
    mu = np.array([0.93, 0.89, 0.85, 0.82, 0.79, 0.76, 0.73])
    c = rng.beta(8 * mu, 8 * (1 - mu), size=(R, g)).astype(np.float32)
    c[::13, 2] = 1.0
    a = O.survival(c)
    sps = sps_table("staircase", R * (1 + g))
    got = O.schedule(a, sps)
    L = got["lengths"]
    sel = np.zeros((R, g), bool)
    for m in range(R):
        sel[m, :L[m]] = True
    if sel.any() and (~sel).any():
        assert a[sel].min() >= a[~sel].max()
    # tau at the chosen budget, recomputed from the lengths
    tau = sum(1 + sum(Fraction(float(a[m, j])) for j in range(L[m])) for m in range(R))
    assert abs(float(tau) - got["tau"]) <= 1e-9 * got["tau"]


def test_staircase_optimum_sits_on_a_plateau_edge():
    rng = np.random.default_rng(6)
    R, g = 200, 7
    a = _rand_surv(rng, R, g)
    sps = sps_table("staircase", R * (1 + g))
    got = O.schedule(a, sps)
    assert got["B_star"] % 512 == 0 or got["B_star"] == R * (1 + g)


def test_budget_shrinks_as_engine_saturates():
    # Load-adaptive behaviour: with SPS(B) = exp(-lam * B), log tau(B) is concave,
    # so the chosen budget is non-increasing in lam.
    rng = np.random.default_rng(7)
    R, g = 64, 6
    a = _rand_surv(rng, R, g)
    B = np.arange(1, R * (1 + g) + 1)
    prev = None
    for lam in [0.0, 1e-4, 1e-3, 3e-3, 1e-2, 3e-2, 1e-1]:
        got = O.schedule(a, np.exp(-lam * B).astype(np.float32))
        if prev is not None:
            assert got["B_star"] <= prev
        prev = got["B_star"]
    assert prev < R * (1 + g)


def test_fixed_point_tau_agrees_with_plain_fp64_sum():
    rng = np.random.default_rng(8)
    a = _rand_surv(rng, 100, 5)
    got = O.schedule(a, sps_table("staircase", 600))
    desc = np.sort(a.reshape(-1).astype(np.float64))[::-1]
    plain = 100 + desc[:got["m_star"]].sum()
    assert abs(plain - got["tau"]) < 1e-9


def test_figure1_keeps_the_confident_prefix():
    with open(os.path.join(GOLDEN, "fig1_prefix.json")) as f:
        fx = json.load(f)
    a = O.survival(np.array(fx["conf"], np.float32))
    sps = (0.97 ** np.arange(0, 8)).astype(np.float32)
    got = O.schedule(a, sps)
    assert list(got["lengths"]) == fx["expected_lengths"]
    B_star, _ = brute_force(a, sps)
    assert got["B_star"] == B_star


def test_equal_survivals_break_ties_by_request_then_position():
    # Every candidate has a = 1/2^j pattern shared across requests: with a
    # budget of K - R = 3 the first three (request, position) pairs in id order
    # among the equal leaders are taken.
    R, g = 4, 2
    a = O.survival(np.full((R, g), 0.5, np.float32))   # a = [0.5, 0.25] in every request
    sps = (np.arange(1, R * (1 + g) + 1) <= R + 3).astype(np.float32)
    got = O.schedule(a, sps)
    assert list(got["lengths"]) == [1, 1, 1, 0]
    assert list(got["order"][:4]) == [0, 2, 4, 6]


def test_theta_ties_take_the_smallest_budget():
    # Zero survivals add nothing to tau; under a constant SPS every budget that
    # only adds them ties, and the smallest one wins.
    a = O.survival(np.array([[0.9, 0.0, 0.0], [0.8, 0.5, 0.0]], np.float32))
    got = O.schedule(a, np.ones(2 * 4, np.float32))
    assert got["m_star"] == 3 and list(got["lengths"]) == [1, 2]


# --------------------------------------------------------------------------- input clamp

def test_survivals_outside_the_unit_interval_are_clamped():
    # Survivals are probabilities: above 1 counts as 1, below 0 and NaN as 0, for
    # the order, q and tau alike.
    rng = np.random.default_rng(17)
    R, g = 30, 4
    a = O.survival(rng.uniform(0.3, 1.0, size=(R, g)).astype(np.float32))
    sps = (0.99 ** np.arange(R * (1 + g))).astype(np.float32)
    raw = a.copy()
    raw[0, 0], raw[3, 1], raw[7, 2], raw[9, 3] = 1.5, np.inf, -0.25, np.nan
    clipped = a.copy()
    clipped[0, 0], clipped[3, 1], clipped[7, 2], clipped[9, 3] = 1.0, 1.0, 0.0, 0.0
    got, want = O.schedule(raw, sps), O.schedule(clipped, sps)
    for k in ("lengths", "order"):
        assert np.array_equal(got[k], want[k])
    assert got["tau_fx"] == want["tau_fx"] and got["m_star"] == want["m_star"]
    # clamped values tie with 1.0 / 0.0 and keep (request, position) order
    order = list(O.candidate_order(raw))
    assert order.index(0 * g + 0) < order.index(3 * g + 1)
    assert order.index(7 * g + 2) < order.index(9 * g + 3)


def test_fixed_point_tau_at_its_largest():
    # With every survival 1, tau_fx after all R * gamma candidates is exactly
    # R (1 + gamma) 2^40: the bound R (1 + gamma) < 2^24 keeps it below 2^64.
    R, g = 7, 3
    a = np.ones((R, g), np.float32)
    B = np.arange(1, R * (1 + g) + 1)
    res = O.schedule(a, np.ones(B.size, np.float32))          # constant SPS: admit all
    assert res["m_star"] == R * g and res["tau_fx"] == R * (1 + g) * (1 << 40)
    assert ((1 << 24) - 1) * (1 << 40) < (1 << 64)
