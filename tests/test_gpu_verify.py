"""GPU parity of the verification side against the CPU oracle.

Flattening and greedy accept / correct are integer work: bit-exact.  The
acceptance probability is a sum over V of fp32 exponentials against the
oracle's fp64 value: |out - ref| <= 2e-5 (each term carries about 1e-7
relative error from expf and the scaling; the fixed-order fp32 sum of up to
~1.3e5 positive terms below 1 adds at most ~1e-6).
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import make_accept_workload, make_verify_workload  # noqa: E402
from oracle import dspark_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ACCEPT_ATOL = 2e-5


def _say(msg):
    print(msg, flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _flatten_target(wl, cu):
    R = wl["R"]
    rows = [wl["target"][r, :cu[r + 1] - cu[r]] for r in range(R)]
    return np.ascontiguousarray(np.concatenate(rows, axis=0))


@pytest.mark.parametrize("R,g", [(1, 1), (5, 4), (1000, 5), (3000, 7)])
def test_verify_pack(R, g):
    _say(f"case verify pack R={R} g={g}")
    wl = make_verify_workload(R, g, V=50000, seed=R)
    ref = O.verify_pack(wl["anchors"], wl["tokens"], wl["lengths"], wl["pos0"])
    ft, fp, fr, cu = D.dspark_verify_pack(_dev(wl["anchors"]), _dev(wl["tokens"]),
                                          _dev(wl["lengths"]), _dev(wl["pos0"]))
    torch.cuda.synchronize()
    B = ref["B"]
    assert np.array_equal(cu.cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(ft.cpu().numpy()[:B], ref["tokens"])
    assert np.array_equal(fp.cpu().numpy()[:B], ref["positions"])
    assert np.array_equal(fr.cpu().numpy()[:B], ref["request"])


def test_verify_pack_without_positions_and_clamped_lengths():
    _say("case verify pack clamp")
    wl = make_verify_workload(40, 3, V=1000, seed=9)
    lengths = wl["lengths"].copy()
    lengths[::7] = 9      # beyond gamma: clamped to gamma
    lengths[1::7] = -2    # below zero: clamped to 0
    ref = O.verify_pack(wl["anchors"], wl["tokens"], np.clip(lengths, 0, 3))
    ft, fp, fr, cu = D.dspark_verify_pack(_dev(wl["anchors"]), _dev(wl["tokens"]), _dev(lengths),
                                          want_pos=True, want_req=False)
    torch.cuda.synchronize()
    assert fr is None
    assert np.array_equal(cu.cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(ft.cpu().numpy()[:ref["B"]], ref["tokens"])
    assert np.array_equal(fp.cpu().numpy()[:ref["B"]], ref["positions"])


@pytest.mark.parametrize("R,g,V,rate", [(1, 4, 37, 1.0), (300, 5, 5000, 0.7), (64, 5, 129280, 0.8),
                                        (17, 16, 4099, 0.9), (200, 3, 1000, 0.0)])
def test_verify_greedy(R, g, V, rate):
    _say(f"case verify greedy R={R} g={g} V={V} rate={rate}")
    wl = make_verify_workload(R, g, V, seed=R + V, match_rate=rate)
    pk = O.verify_pack(wl["anchors"], wl["tokens"], wl["lengths"])
    tl = _flatten_target(wl, pk["cu_seqlens"])
    ref = O.verify_greedy(tl, pk["cu_seqlens"], wl["tokens"], wl["lengths"])
    acc, nxt, amax = D.dspark_verify_greedy(_dev(tl), _dev(pk["cu_seqlens"]), _dev(wl["tokens"]))
    torch.cuda.synchronize()
    B = pk["B"]
    assert np.array_equal(amax.cpu().numpy()[:B], ref["target_argmax"])
    assert np.array_equal(acc.cpu().numpy(), ref["accepted"])
    assert np.array_equal(nxt.cpu().numpy(), ref["next_token"])
    if rate == 1.0:
        assert np.array_equal(acc.cpu().numpy(), wl["lengths"])


def test_verify_greedy_ties_take_the_smallest_id():
    _say("case verify greedy ties")
    R, g, V = 8, 3, 1024
    wl = make_verify_workload(R, g, V, seed=3, match_rate=0.0)
    pk = O.verify_pack(wl["anchors"], wl["tokens"], wl["lengths"])
    tl = _flatten_target(wl, pk["cu_seqlens"])
    rng = np.random.default_rng(4)
    for e in range(tl.shape[0]):
        ids = rng.choice(V, size=3, replace=False)
        tl[e, ids] = tl[e].max() + 2.0
    ref = O.verify_greedy(tl, pk["cu_seqlens"], wl["tokens"], wl["lengths"])
    acc, nxt, amax = D.dspark_verify_greedy(_dev(tl), _dev(pk["cu_seqlens"]), _dev(wl["tokens"]))
    torch.cuda.synchronize()
    assert np.array_equal(amax.cpu().numpy()[:pk["B"]], ref["target_argmax"])
    assert np.array_equal(nxt.cpu().numpy(), ref["next_token"])


# Aligned rows of a multiple of four entries take the holding kernel: 512
# threads keep 24 groups of four entries each in registers (49152 entries per
# row) and 8 more in LDS (65536 in all) between the passes; the rest is read
# twice.  The cases put V below, at and just past those boundaries; 4099 takes
# the other kernel.
@pytest.mark.parametrize("n,V,T", [(64, 4099, 1.0), (64, 4096, 0.7), (37, 129280, 1.0),
                                   (8, 151936, 1.3), (16, 49152, 1.0), (16, 49156, 0.9),
                                   (16, 65532, 1.1), (16, 65536, 1.0), (16, 65540, 0.8)])
def test_accept_prob(n, V, T):
    _say(f"case accept prob n={n} V={V} T={T}")
    wl = make_accept_workload(n, V, seed=n + V)
    ref = O.accept_prob(wl["draft"], wl["target"], T)
    got = D.dspark_accept_prob(_dev(wl["draft"]), _dev(wl["target"]), T).cpu().numpy()
    assert np.abs(got.astype(np.float64) - ref).max() <= ACCEPT_ATOL


def test_accept_prob_special_rows_across_held_regions():
    # The special rows at V = 70000: identical, unrelated, disjoint supports
    # split inside the LDS-held region, and a mask of every third entry.
    _say("case accept prob special rows across the held regions")
    V = 70000
    rng = np.random.default_rng(6)
    d = rng.normal(size=(4, V)).astype(np.float32)
    t = d.copy()
    t[1] = rng.normal(size=V)
    d[2, 60000:] = -np.inf
    t[2, :60000] = -np.inf
    d[3, ::3] = -np.inf
    ref = O.accept_prob(d, t)
    got = D.dspark_accept_prob(_dev(d), _dev(t)).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.abs(got.astype(np.float64) - ref).max() <= ACCEPT_ATOL
    assert abs(got[0] - 1.0) <= ACCEPT_ATOL and got[2] == 0.0


def test_accept_prob_special_rows():
    _say("case accept prob special rows")
    V = 1000
    rng = np.random.default_rng(5)
    d = rng.normal(size=(4, V)).astype(np.float32)
    t = d.copy()                              # row 0: identical -> 1
    t[1] = rng.normal(size=V)                 # row 1: unrelated
    d[2, 500:] = -np.inf                      # row 2: disjoint supports -> 0
    t[2, :500] = -np.inf
    d[3, ::2] = -np.inf                       # row 3: partial masks
    ref = O.accept_prob(d, t)
    got = D.dspark_accept_prob(_dev(d), _dev(t)).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.abs(got.astype(np.float64) - ref).max() <= ACCEPT_ATOL
    assert abs(got[0] - 1.0) <= ACCEPT_ATOL and got[2] == 0.0
