"""Pins for the oracle's two other admission rules (CPU only).

* Early stop ([P1] §二 设计二, greedy steps 3-5): candidates are admitted one at
  a time in sorted order and the scan stops as soon as Theta no longer
  increases.  Pinned by a worked example, by the SPS curves where it must agree
  with the global search (it agrees whenever Theta is unimodal in m), by the
  non-anticipation property the pages give for the break (the decision depends
  only on the prefix processed so far), and by a staircase case where it stops
  at the first plateau edge while the global search goes further.
* Capacity K ([P1] §三 挑战1, [P3] part 01): the top K - R candidates by current
  survival.  Pinned by brute-force selection and by the global search with a
  step SPS, which the scheduler's own pins tie to the same top-K set.
"""
import numpy as np
import pytest

from oracle import dspark_oracle as O
from draft_head_step_amd.inputs import sps_table


def _rand_surv(rng, R, g, lo=0.05):
    return O.survival(rng.uniform(lo, 1.0, size=(R, g)).astype(np.float32))


# ----------------------------------------------------------------- early stop

def test_early_stop_worked_example():
    # a (exact binary fractions): request 0: 0.5, 0.25; request 1: 0.75, 0.125.
    # Sorted: 0.75 (id 2), 0.5 (id 0), 0.25 (id 1), 0.125 (id 3), so
    # tau_m = 2, 2.75, 3.25, 3.5, 3.625 for m = 0..4 and B = 2 + m.
    # SPS: B=2 -> 1.0, B=3..6 -> 0.75 (a one-step drop, then flat).
    # Theta_m = 2.0, 2.0625, 2.4375, 2.625, 2.71875: strictly increasing, so the
    # early stop admits everything, like the global search.
    a = np.array([[0.5, 0.25], [0.75, 0.125]], np.float32)
    sps = np.array([1.0, 1.0, 0.75, 0.75, 0.75, 0.75], np.float32)
    got = O.schedule_early_stop(a, sps)
    assert got["m_star"] == 4 and list(got["lengths"]) == [2, 2]
    assert got["theta"] == 3.625 * 0.75
    # Now SPS(3) = 0.5: Theta_1 = 2.75 * 0.5 = 1.375 <= Theta_0 = 2, so the scan
    # stops before the first candidate, while Theta_4 = 3.625 * 0.75 = 2.71875 is
    # the global maximum.
    sps2 = np.array([1.0, 1.0, 0.5, 0.75, 0.75, 0.75], np.float32)
    es = O.schedule_early_stop(a, sps2)
    gl = O.schedule(a, sps2)
    assert es["m_star"] == 0 and es["B_star"] == 2 and list(es["lengths"]) == [0, 0]
    assert es["tau_fx"] == 2 << 40 and es["theta"] == 2.0
    assert gl["m_star"] == 4
    # Equal Theta counts as "no longer increasing": with a top survival of 1.0,
    # tau_1 = 3, and SPS(2) = 0.75, SPS(3) = 0.5 give Theta_0 = 2 * 0.75 = 1.5 =
    # Theta_1 = 3 * 0.5 exactly.
    a3 = np.array([[1.0, 0.5], [0.25, 0.125]], np.float32)
    sps3 = np.array([1.0, 0.75, 0.5, 0.5, 0.5, 0.5], np.float32)
    es3 = O.schedule_early_stop(a3, sps3)
    assert es3["m_star"] == 0 and es3["theta"] == 1.5


def test_early_stop_constant_sps_takes_every_positive_candidate():
    rng = np.random.default_rng(31)
    a = _rand_surv(rng, 20, 6)
    sps = np.ones(20 * 7, np.float32)
    es = O.schedule_early_stop(a, sps)
    assert es["m_star"] == 120 == O.schedule(a, sps)["m_star"]
    assert np.all(es["lengths"] == 6)


def test_early_stop_reciprocal_sps_takes_nothing():
    rng = np.random.default_rng(32)
    a = O.survival(rng.uniform(0.05, 0.99, size=(9, 4)).astype(np.float32))
    B = np.arange(1, 9 * 5 + 1)
    assert O.schedule_early_stop(a, (1.0 / B).astype(np.float32))["m_star"] == 0


@pytest.mark.parametrize("K", [7, 20, 33])
def test_early_stop_step_sps_is_top_k(K):
    rng = np.random.default_rng(100 + K)
    R, g = 6, 5
    a = _rand_surv(rng, R, g)
    sps = (np.arange(1, R * (1 + g) + 1) <= K).astype(np.float32)
    es = O.schedule_early_stop(a, sps)
    gl = O.schedule(a, sps)
    assert es["B_star"] == K == gl["B_star"]
    assert np.array_equal(es["lengths"], gl["lengths"]) and es["tau_fx"] == gl["tau_fx"]


@pytest.mark.parametrize("R,g,slope,seed", [(8, 5, 0.01, 1), (40, 4, 0.002, 2), (100, 7, 0.0005, 3),
                                            (300, 5, 0.0001, 4)])
def test_early_stop_equals_global_search_when_theta_is_unimodal(R, g, slope, seed):
    # With a linear decreasing SPS, Theta_{m+1} - Theta_m = a_{m+1} s_{m+1} - tau_m (s_m - s_{m+1})
    # decreases in m (a and s fall, tau rises), so Theta rises then falls and the
    # first break is the global maximum -- up to the fp32 rounding of the SPS
    # table, which can make a tiny local maximum right at the peak (it does at
    # R = 3000, slope 2e-5: m* 9123 against 9127); these cases have none.
    rng = np.random.default_rng(seed)
    a = _rand_surv(rng, R, g)
    B = np.arange(1, R * (1 + g) + 1, dtype=np.float64)
    sps = np.maximum(1.0 - slope * (B - 1), 1e-3).astype(np.float32)
    es = O.schedule_early_stop(a, sps)
    gl = O.schedule(a, sps)
    assert es["m_star"] == gl["m_star"]
    assert es["tau_fx"] == gl["tau_fx"] and es["theta"] == gl["theta"]
    assert np.array_equal(es["lengths"], gl["lengths"])


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_early_stop_does_not_look_past_its_break(seed):
    # Non-anticipation: the break depends only on the candidates up to the first
    # one it rejects, so lowering every later survival (keeping the order and
    # staying positive) leaves the decision unchanged.
    rng = np.random.default_rng(seed)
    R, g = 50, 5
    a = _rand_surv(rng, R, g)
    sps = sps_table("staircase", R * (1 + g))
    B = np.arange(1, R * (1 + g) + 1, dtype=np.float64)
    sps = (sps * np.maximum(1.0 - 0.002 * (B - 1), 0.05)).astype(np.float32)
    es = O.schedule_early_stop(a, sps)
    m = es["m_star"]
    order = es["order"]
    assert m < R * g
    flat = a.reshape(-1).copy()
    cut = float(flat[order[m]])
    later = order[m + 1:]
    flat[later] = np.minimum(flat[later], cut) * np.float32(0.5)
    b = flat.reshape(R, g)
    assert np.array_equal(O.candidate_order(b)[:m + 1], order[:m + 1])
    es2 = O.schedule_early_stop(b, sps)
    assert es2["m_star"] == m and np.array_equal(es2["lengths"], es["lengths"])


def test_early_stop_stops_at_the_first_plateau_edge_of_the_staircase():
    # Staircase SPS (plateaus of 512 budgets, 3% lower each): inside a plateau
    # Theta grows with every positive candidate; at B = 513 it falls by 3% while
    # one candidate adds at most 1/tau ~ 0.2% (tau >= R = 512), so the early stop
    # stops at B = 512.  The global search keeps going: with survivals near 1 the
    # plateaus further right hold more tau than the 3% steps take away.
    rng = np.random.default_rng(8)
    R, g = 512, 7
    a = O.survival(rng.uniform(0.97, 1.0, size=(R, g)).astype(np.float32))
    sps = sps_table("staircase", R * (1 + g))
    es = O.schedule_early_stop(a, sps)
    gl = O.schedule(a, sps)
    assert es["B_star"] == 512 and es["m_star"] == 0
    # The first plateau edge is B = 512 = R: the first candidate already costs 3%.
    assert gl["B_star"] > es["B_star"]
    assert gl["theta"] > es["theta"]
    # R = 256: the first plateau (B <= 512) admits 256 candidates before the break.
    a2 = O.survival(rng.uniform(0.97, 1.0, size=(256, 7)).astype(np.float32))
    sps2 = sps_table("staircase", 256 * 8)
    es2 = O.schedule_early_stop(a2, sps2)
    gl2 = O.schedule(a2, sps2)
    assert es2["B_star"] == 512 and es2["m_star"] == 256
    assert gl2["B_star"] > 512 and gl2["theta"] > es2["theta"]


# ----------------------------------------------------------------- capacity K

@pytest.mark.parametrize("R,g,K,seed", [(6, 5, 7, 1), (6, 5, 20, 2), (6, 5, 36, 3), (40, 3, 100, 4),
                                        (40, 3, 10, 5), (40, 3, 1000, 6)])
def test_capacity_is_brute_force_top_k(R, g, K, seed):
    rng = np.random.default_rng(seed)
    a = _rand_surv(rng, R, g)
    got = O.schedule_capacity(a, K)
    m = min(max(K - R, 0), R * g)
    flat = a.reshape(-1)
    ids = sorted(range(R * g), key=lambda i: (-float(flat[i]), i))[:m]
    want = np.bincount(np.array(ids, dtype=np.int64) // g, minlength=R)
    assert got["m_star"] == m and got["B_star"] == R + m
    assert np.array_equal(got["lengths"], want)
    tau = R + sum(float(np.float64(flat[i])) for i in ids)
    assert abs(got["tau"] - tau) <= 1e-9 * tau


@pytest.mark.parametrize("K", [9, 21, 30])
def test_capacity_equals_global_search_with_step_sps(K):
    rng = np.random.default_rng(200 + K)
    R, g = 6, 5
    a = _rand_surv(rng, R, g)
    sps = (np.arange(1, R * (1 + g) + 1) <= K).astype(np.float32)
    cap = O.schedule_capacity(a, K)
    gl = O.schedule(a, sps)
    for k in ("m_star", "B_star", "tau_fx", "tau"):
        assert cap[k] == gl[k]
    assert np.array_equal(cap["lengths"], gl["lengths"])
    assert cap["theta"] == cap["tau"]


def test_capacity_takes_exactly_k_even_with_zero_survivals():
    # Zero survivals add nothing to tau, so the global search with a step SPS
    # stops before them (first argmax); the capacity rule fills the batch anyway.
    a = np.array([[1.0, 0.0], [0.5, 0.0]], np.float32)
    cap = O.schedule_capacity(a, 6)
    assert cap["m_star"] == 4 and list(cap["lengths"]) == [2, 2]
    sps = (np.arange(1, 7) <= 6).astype(np.float32)
    assert O.schedule(a, sps)["m_star"] == 2
