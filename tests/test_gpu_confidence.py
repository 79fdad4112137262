"""GPU parity of the confidence head (dspark_confidence, and the fused step's
prologue that computes the same token-independent part) at shapes that take
each kernel path: one or two 16-byte pieces of h per thread, positions in
several rounds, the general kernel for d not a multiple of 8 or d above
16384, and a single position.

Confidences within 1e-4 of the oracle, survival bit-exact given the GPU's
confidences (the bars stated in gpu_helpers); an invalid token gives NaN at
its position and in every later survival.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import GREEDY, Config, make_workload  # noqa: E402
from oracle import dspark_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # name, R, gamma, V, r, d
    ("two_pieces_three_rounds", 6, 11, 2048, 128, 12288),   # 1536 pieces: two per thread, G = 4
    ("two_pieces_one_extra", 3, 4, 1024, 64, 8200),         # 1025 pieces: one second piece
    ("one_piece_full", 5, 9, 1024, 512, 8192),              # 1024 pieces, two rounds of G = 8
    ("general_d", 4, 3, 1024, 48, 260),                     # d % 8 != 0: general kernel
    ("general_big_d", 2, 2, 512, 16, 16392),                # 2049 pieces: general kernel
    ("one_position", 7, 1, 512, 16, 64),
]


def _say(msg):
    print(msg, flush=True)


def _workload(name, R, g, V, r, d):
    cfg = Config(name, R=R, gamma=g, V=V, r=r, d=d, mode=GREEDY, w_std=0.2, base_std=1.0,
                 wconf_std=0.05, sts=tuple(1.0 + 0.1 * k for k in range(g)), seed=700 + d)
    wl = make_workload(cfg)
    tokens = np.random.default_rng(d).integers(0, V, size=(R, g), dtype=np.int32)
    return wl, tokens


@pytest.mark.parametrize("name,R,g,V,r,d", CASES)
def test_confidence_paths_match_oracle(name, R, g, V, r, d):
    _say(f"case confidence {name} R={R} g={g} V={V} r={r} d={d}")
    wl, tokens = _workload(name, R, g, V, r, d)
    dev = H.to_device(wl, DEV)
    conf, surv = H.run_confidence(wl, dev, torch.from_numpy(tokens).to(DEV))
    H.check_confidence(wl, tokens, conf, surv)


@pytest.mark.parametrize("name,R,g,V,r,d", CASES)
def test_confidence_invalid_token_gives_nan(name, R, g, V, r, d):
    _say(f"case confidence invalid token {name}")
    wl, tokens = _workload(name, R, g, V, r, d)
    bad_m, bad_k = R - 1, g - 1          # x_{g-1} of the last request is read at position g-1
    if g > 1:
        tokens[bad_m, bad_k - 1] = V      # one past the vocabulary
    anchors = wl["anchors"].copy()
    if g == 1:
        anchors[bad_m] = -3
    dev = H.to_device(wl, DEV)
    conf, surv = D.dspark_confidence(dev["h"], dev["W1"], torch.from_numpy(anchors).to(DEV),
                                     torch.from_numpy(tokens).to(DEV), dev["w_conf"], dev["sts"])
    torch.cuda.synchronize()
    c, s = conf.cpu().numpy(), surv.cpu().numpy()
    assert np.isnan(c[bad_m, bad_k]) and np.isnan(s[bad_m, bad_k:]).all()
    ok = np.ones_like(c, dtype=bool)
    ok[bad_m, bad_k] = False
    assert not np.isnan(c[ok]).any()
    safe = tokens.copy()
    safe[bad_m] = 0
    ref = O.confidence(wl["h"], wl["W1"], wl["anchors"], safe, wl["w_conf"], wl["sts"])
    keep = np.ones(R, dtype=bool)
    keep[bad_m] = False
    assert np.abs(c[keep].astype(np.float64) - ref[keep]).max() <= H.CONF_ATOL


@pytest.mark.parametrize("name,R,g,V,r,d", [c for c in CASES if c[5] % 4 == 0])
def test_fused_step_prologue_paths(name, R, g, V, r, d):
    # The fused step computes w_h . h in its prologue (the same row kernels) and
    # adds the embedding term from the step kernels.
    _say(f"case fused prologue {name}")
    wl, _ = _workload(name, R, g, V, r, d)
    dev = H.to_device(wl, DEV)
    tok, conf, surv, lengths, order, info = D.dspark_draft_step(
        dev["W1"], dev["W2"], dev["base"], dev["anchors"], dev["h"], dev["w_conf"], dev["sps"],
        GREEDY, 1.0, None, sts_temp=dev["sts"], want_order=True, want_info=True)
    torch.cuda.synchronize()
    toks = tok.cpu().numpy()
    H.check_draft(wl, toks)
    H.check_confidence(wl, toks, conf.cpu().numpy(), surv.cpu().numpy())
    H.check_schedule(surv.cpu().numpy(), wl["sps"], lengths.cpu().numpy(), order.cpu().numpy(),
                     D.schedule_info(info))
