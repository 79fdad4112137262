"""Pins for the oracle's verification side (CPU only).

* verify_pack / verify_greedy: the Figure 1 round of [P3] worked by hand
  (prompt ABC, anchor D, drafts EFGH, the scheduler keeps EFG, the target
  accepts E and F, rejects G and emits G*), the all-accepted and
  first-rejected cases, and the flattening invariants.
* accept_prob: closed forms (identical and disjoint distributions, two-point
  distributions), the identity sum_v min(p, q) = 1 - (1/2) sum_v |p - q|
  evaluated independently, and invariance to adding a constant to the logits.
"""
import numpy as np
import pytest

from oracle import dspark_oracle as O

A, B_, C, D, E, F, G, H, G_STAR = range(9)   # token ids of Figure 1 (G* != G)


def _onehot_rows(ids, V, hi=5.0):
    z = np.zeros((len(ids), V), np.float32)
    z[np.arange(len(ids)), ids] = hi
    return z


def test_figure1_round():
    # Prompt ABC occupies positions 0..2, so the anchor D sits at position 3.
    drafts = np.array([[E, F, G, H]], np.int32)
    pk = O.verify_pack(np.array([D], np.int32), drafts, np.array([3]), pos0=np.array([3]))
    assert pk["B"] == 4 and list(pk["cu_seqlens"]) == [0, 4]
    assert list(pk["tokens"]) == [D, E, F, G]          # H was dropped by the scheduler
    assert list(pk["positions"]) == [3, 4, 5, 6]
    assert list(pk["request"]) == [0, 0, 0, 0]
    # The target's next token after D, E, F, G: E, F, G*, (anything).
    tl = _onehot_rows([E, F, G_STAR, A], V=12)
    vg = O.verify_greedy(tl, pk["cu_seqlens"], drafts, np.array([3]))
    assert vg["accepted"][0] == 2                      # E and F
    assert vg["next_token"][0] == G_STAR               # the corrected token


def test_greedy_all_accepted_takes_the_bonus_token_and_zero_length_takes_the_targets():
    drafts = np.array([[4, 5, 6], [7, 8, 9]], np.int32)
    lengths = np.array([3, 0])
    pk = O.verify_pack(np.array([1, 2], np.int32), drafts, lengths)
    assert list(pk["cu_seqlens"]) == [0, 4, 5]
    # request 0: target agrees with every draft, bonus 10; request 1: only its anchor
    tl = _onehot_rows([4, 5, 6, 10, 11], V=16)
    vg = O.verify_greedy(tl, pk["cu_seqlens"], drafts, lengths)
    assert list(vg["accepted"]) == [3, 0] and list(vg["next_token"]) == [10, 11]


def test_greedy_first_draft_rejected():
    drafts = np.array([[4, 5]], np.int32)
    tl = _onehot_rows([3, 5, 6], V=8)                  # 3 != 4: nothing accepted
    vg = O.verify_greedy(tl, np.array([0, 3]), drafts, np.array([2]))
    assert vg["accepted"][0] == 0 and vg["next_token"][0] == 3


def test_greedy_target_ties_take_the_smallest_id():
    z = np.zeros((2, 6), np.float32)
    z[0, [2, 4]] = 1.0                                 # tie between 2 and 4 -> 2
    z[1, 5] = 1.0
    vg = O.verify_greedy(z, np.array([0, 2]), np.array([[2]], np.int32), np.array([1]))
    assert vg["target_argmax"][0] == 2 and vg["accepted"][0] == 1 and vg["next_token"][0] == 5


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_invariants(seed):
    rng = np.random.default_rng(seed)
    R, g = 37, 6
    anchors = rng.integers(0, 1000, size=R).astype(np.int32)
    drafts = rng.integers(0, 1000, size=(R, g)).astype(np.int32)
    lengths = rng.integers(0, g + 1, size=R)
    pos0 = rng.integers(0, 5000, size=R)
    pk = O.verify_pack(anchors, drafts, lengths, pos0)
    cu = pk["cu_seqlens"]
    assert pk["B"] == R + int(lengths.sum()) == cu[-1]
    assert np.all(np.diff(cu) == 1 + lengths)
    for r in range(R):
        seg = slice(cu[r], cu[r + 1])
        assert pk["tokens"][cu[r]] == anchors[r]
        assert np.array_equal(pk["tokens"][cu[r] + 1:cu[r + 1]], drafts[r, :lengths[r]])
        assert np.array_equal(pk["positions"][seg], pos0[r] + np.arange(1 + lengths[r]))
        assert np.all(pk["request"][seg] == r)


def test_accept_prob_closed_forms():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(4, 50)).astype(np.float32)
    assert np.allclose(O.accept_prob(z, z), 1.0, atol=1e-12)
    # disjoint supports
    zd = np.full((1, 6), -np.inf, np.float32)
    zt = np.full((1, 6), -np.inf, np.float32)
    zd[0, :3] = 0.0
    zt[0, 3:] = 0.0
    assert O.accept_prob(zd, zt)[0] == 0.0
    # two-point distributions: p = (a, 1 - a), q = (b, 1 - b) -> 1 - |a - b|
    for a, b in [(0.2, 0.7), (0.5, 0.5), (0.9, 0.1), (0.01, 0.02)]:
        ld = np.log(np.array([[a, 1 - a]]))
        lt = np.log(np.array([[b, 1 - b]]))
        assert abs(O.accept_prob(ld, lt)[0] - (1.0 - abs(a - b))) < 1e-12


def test_accept_prob_is_one_minus_total_variation():
    rng = np.random.default_rng(6)
    zd = rng.normal(scale=2.0, size=(5, 300))
    zt = zd + rng.normal(scale=0.5, size=(5, 300))
    got = O.accept_prob(zd, zt)
    for i in range(5):
        p = np.exp(zd[i] - zd[i].max())
        p /= p.sum()
        q = np.exp(zt[i] - zt[i].max())
        q /= q.sum()
        tv = 0.5 * sum(abs(float(x) - float(y)) for x, y in zip(p, q))
        assert abs(got[i] - (1.0 - tv)) < 1e-12


def test_accept_prob_shift_and_temperature():
    rng = np.random.default_rng(7)
    zd = rng.normal(size=(3, 80))
    zt = rng.normal(size=(3, 80))
    base = O.accept_prob(zd, zt)
    assert np.allclose(O.accept_prob(zd + 3.0, zt - 7.0), base, atol=1e-12)
    # a very high temperature flattens both toward uniform
    assert np.all(O.accept_prob(zd, zt, temperature=1e6) > 1 - 1e-5)
    # temperature T equals scaling the logits by 1/T
    assert np.allclose(O.accept_prob(zd, zt, temperature=0.5), O.accept_prob(2 * zd, 2 * zt),
                       atol=1e-12)
