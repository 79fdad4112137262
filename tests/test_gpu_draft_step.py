"""GPU parity of the fused draft step (dspark_draft_step: draft, confidence +
STS + survival, schedule in one call) and of the device-side id checks.

The fused call is compared with the CPU oracle to the bars stated in
gpu_helpers (tokens on the forced sequence, confidences within 1e-4,
survival and schedule bit-exact given the GPU's confidences), and its tokens
with those of dspark_markov_draft on the same inputs (the same step kernels:
bit-identical).
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import CONFIGS, GREEDY, SAMPLE, Config, make_workload, to_tiled  # noqa: E402
from oracle import dspark_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _tile_rows(R, per_tile, seed):
    rng = np.random.default_rng(seed)
    rows = [0, R - 1]
    for t0 in range(0, R, 32):
        n = min(32, R - t0)
        rows += list(t0 + rng.choice(n, size=min(per_tile, n), replace=False))
    return np.unique(np.asarray(rows))


def _fused(wl, g, layout):
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(DEV)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(DEV)
    else:
        base, unif = g["base"], g.get("uniforms")
    out = D.dspark_draft_step(g["W1"], g["W2"], base, g["anchors"], g["h"], g["w_conf"], g["sps"],
                              wl["mode"], wl["temperature"], unif, sts_temp=g.get("sts"),
                              want_order=True, want_info=True, layout=layout)
    ref_tok = D.dspark_markov_draft(g["W1"], g["W2"], base, g["anchors"], wl["mode"],
                                    wl["temperature"], unif, layout=layout)
    torch.cuda.synchronize()
    return out, ref_tok


def _check_fused(wl, layout, rows=None):
    g = H.to_device(wl, DEV)
    (tok, conf, surv, lengths, order, info), ref_tok = _fused(wl, g, layout)
    toks = tok.cpu().numpy()
    assert np.array_equal(toks, ref_tok.cpu().numpy()), "fused tokens differ from dspark_markov_draft"
    H.check_draft(wl, toks, rows)
    H.check_confidence(wl, toks, conf.cpu().numpy(), surv.cpu().numpy())
    H.check_schedule(surv.cpu().numpy(), wl["sps"], lengths.cpu().numpy(), order.cpu().numpy(),
                     D.schedule_info(info))


CASES = [
    # name, R, gamma, V, r, d, mode
    ("tiny", 4, 5, 4096, 64, 256, GREEDY),
    ("r48", 33, 3, 1001, 48, 40, SAMPLE),
    ("r256", 70, 4, 3000, 256, 100, SAMPLE),
    ("r512s", 40, 3, 5000, 512, 64, SAMPLE),
    ("r512g", 300, 2, 3000, 512, 16, GREEDY),
    ("global", 2000, 5, 2000, 64, 32, GREEDY),    # 10000 candidates: the schedule's global path
    ("g1", 50, 1, 3000, 64, 16, SAMPLE),          # one position: prologue, one step, finish
    ("g16", 20, 16, 2000, 128, 24, GREEDY),       # a long block of sixteen positions
]


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("name,R,g,V,r,d,mode", CASES)
def test_draft_step_matches_oracle(name, R, g, V, r, d, mode, layout):
    _say(f"case draft_step {name} R={R} g={g} V={V} r={r} d={d} mode={mode} layout={layout}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=0.9, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, sts=tuple(1.0 + 0.1 * k for k in range(g)),
                 seed=300 + R)
    _check_fused(make_workload(cfg), layout, None if R <= 300 else _tile_rows(R, 1, R))


# Rank-512 sampling runs on the K-split kernel, whose last step does the
# finishing work on a workgroup without step work when it has one and
# R gamma <= 4 x its threads (gamma + 1 launches); else a launch follows the
# last step (gamma + 2).  launches: the count the library reports for the
# row-major layout on MI355X.
FIN_CASES = [
    # name, R, gamma, V, r, d, launches
    ("fin_g1", 64, 1, 5000, 512, 64, 2),         # x_{-1} is the anchor
    ("fin_two_blocks", 70, 3, 3000, 384, 48, 4),  # R block 0 of two
    ("fin_at_limit", 100, 20, 4000, 512, 32, 21),  # 2000 candidates, 512 threads x 4
    ("fin_past_limit", 100, 21, 4000, 512, 32, 23),  # 2100: the launch after the last step
    ("fin_one_wave", 20, 6, 2600, 512, 16, 7),    # 128 threads
]


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("name,R,g,V,r,d,launches", FIN_CASES)
def test_draft_step_finishing_in_last_step(name, R, g, V, r, d, launches, layout):
    _say(f"case draft_step {name} R={R} g={g} V={V} r={r} layout={layout}")
    if layout == D.LAYOUT_RGV:
        assert D.dspark_draft_step_launches(R, g, V, r, layout, SAMPLE, 0.8) == launches
    cfg = Config("fin", R=R, gamma=g, V=V, r=r, d=d, mode=SAMPLE, temperature=0.8, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, sts=tuple(1.0 + 0.05 * k for k in range(g)),
                 seed=500 + R + g)
    _check_fused(make_workload(cfg), layout)


def test_draft_step_launch_counts():
    # The DeepSeek-V4 shape: the last step's spare workgroup (127 V groups in a
    # launch of 128) does the finishing work; the tiled layout's strided groups
    # fill the launch, and rank 256 greedy runs the plain kernel.
    dsv4 = (256, 5, 129280, 512)
    assert D.dspark_draft_step_launches(*dsv4, D.LAYOUT_RGV, SAMPLE, 1.0) == 6
    assert D.dspark_draft_step_launches(*dsv4, D.LAYOUT_TILED, SAMPLE, 1.0) == 7
    assert D.dspark_draft_step_launches(64, 5, 151936, 256, D.LAYOUT_RGV, GREEDY, 1.0) == 7
    # 16384 candidates: a finishing launch, then the schedule's global path
    # (four passes of histogram + scatter, then three).
    assert D.dspark_draft_step_launches(1024, 16, 129280, 256, D.LAYOUT_RGV, GREEDY, 1.0) == 29


def test_draft_step_finishing_in_last_step_bad_anchors():
    # Bad anchors on the in-step path: -1 tokens, NaN confidences (also at the
    # last position, whose embedding term the finishing workgroup computes
    # itself), survivals taken as 0 by the schedule.
    _say("case draft_step finishing in last step, bad anchors")
    cfg = Config("edge", R=70, gamma=3, V=3000, r=512, d=32, mode=SAMPLE, temperature=1.1,
                 w_std=0.2, base_std=1.0, wconf_std=0.1, seed=77)
    wl = make_workload(cfg)
    assert D.dspark_draft_step_launches(70, 3, 3000, 512, D.LAYOUT_RGV, SAMPLE, 1.1) == 4
    bad = np.array([0, 5, 33, 69])
    anchors = wl["anchors"].copy()
    anchors[bad] = np.array([-1, 3000, 1 << 30, -(1 << 31)], np.int32)
    g = H.to_device(wl, DEV)
    tok, conf, surv, lengths, order, info = D.dspark_draft_step(
        g["W1"], g["W2"], g["base"], torch.from_numpy(anchors).to(DEV), g["h"], g["w_conf"],
        g["sps"], SAMPLE, 1.1, g["uniforms"], want_order=True, want_info=True)
    torch.cuda.synchronize()
    t, c, s = tok.cpu().numpy(), conf.cpu().numpy(), surv.cpu().numpy()
    assert np.all(t[bad] == -1) and np.all(np.isnan(c[bad])) and np.all(np.isnan(s[bad]))
    keep = np.setdiff1d(np.arange(70), bad)
    assert not np.isnan(c[keep]).any()
    H.check_schedule(s, wl["sps"], lengths.cpu().numpy(), order.cpu().numpy(), D.schedule_info(info))
    assert np.all(lengths.cpu().numpy()[bad] == 0)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_draft_step_qwen3_8b_full(layout):
    _say(f"case draft_step qwen3_8b layout={layout}")
    _check_fused(make_workload(CONFIGS["qwen3_8b"]), layout)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_draft_step_dsv4_full(layout):
    _say(f"case draft_step dsv4 layout={layout}")
    _check_fused(make_workload(CONFIGS["dsv4"]), layout, _tile_rows(256, 3, 7))


def test_draft_step_dirty_workspace_and_repeat():
    # A workspace full of 0xff gives the same results, and so does a second call.
    _say("case draft_step dirty workspace")
    cfg = dataclasses.replace(CONFIGS["tiny"], mode=SAMPLE, temperature=0.8)
    wl = make_workload(cfg, w_std=0.3)
    g = H.to_device(wl, DEV)
    R, gm, V = wl["base"].shape
    ws = torch.full((D.dspark_draft_step_workspace(R, gm, V, wl["r"]),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    outs = []
    for _ in range(2):
        o = D.dspark_draft_step(g["W1"], g["W2"], g["base"], g["anchors"], g["h"], g["w_conf"],
                                g["sps"], SAMPLE, 0.8, g["uniforms"], workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in o[:4]])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    H.check_draft(wl, outs[0][0])


# --------------------------------------------------------------------------- id checks

def _bad_anchor_workload(layout_seed=0):
    cfg = Config("edge", R=70, gamma=3, V=3000, r=64, d=32, mode=GREEDY, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, seed=55 + layout_seed)
    wl = make_workload(cfg)
    bad = np.array([0, 5, 33, 69])
    anchors = wl["anchors"].copy()
    anchors[bad] = np.array([-1, 3000, 1 << 30, -(1 << 31)], np.int32)
    return wl, anchors, bad


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_bad_anchors_give_minus_one(layout):
    # Requests whose anchor is outside [0, V) draft -1 at every position; the
    # other requests are drafted exactly as with valid anchors.
    _say(f"case bad anchors layout={layout}")
    wl, anchors, bad = _bad_anchor_workload()
    g = H.to_device(wl, DEV)
    base = g["base"] if layout == D.LAYOUT_RGV else torch.from_numpy(to_tiled(wl["base"])).to(DEV)
    tok = D.dspark_markov_draft(g["W1"], g["W2"], base, torch.from_numpy(anchors).to(DEV), GREEDY,
                                layout=layout).cpu().numpy()
    good = D.dspark_markov_draft(g["W1"], g["W2"], base, g["anchors"], GREEDY,
                                 layout=layout).cpu().numpy()
    assert np.all(tok[bad] == -1)
    keep = np.setdiff1d(np.arange(wl["R"]), bad)
    assert np.array_equal(tok[keep], good[keep])
    # the confidence head gives NaN from the bad position on
    conf, surv = D.dspark_confidence(g["h"], g["W1"], torch.from_numpy(anchors).to(DEV),
                                     torch.from_numpy(tok).to(DEV), g["w_conf"])
    c, s = conf.cpu().numpy(), surv.cpu().numpy()
    assert np.all(np.isnan(c[bad])) and np.all(np.isnan(s[bad]))
    assert not np.isnan(c[keep]).any()


def test_bad_token_mid_chain_gives_nan_confidence():
    _say("case bad token mid-chain")
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    tok = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], GREEDY).cpu().numpy()
    tok[1, 2] = wl["V"] + 7          # x_3 of request 1: positions 4 and 5 use it
    conf, surv = D.dspark_confidence(g["h"], g["W1"], g["anchors"], torch.from_numpy(tok).to(DEV),
                                     g["w_conf"])
    c, s = conf.cpu().numpy(), surv.cpu().numpy()
    assert np.isnan(c[1, 3]) and not np.isnan(c[1, :3]).any() and np.isnan(s[1, 3:]).all()
    ref = O.confidence(wl["h"], wl["W1"], wl["anchors"], np.where(tok < wl["V"], tok, 0),
                       wl["w_conf"])
    ok = ~np.isnan(c)
    assert np.abs(c[ok] - ref[ok]).max() <= H.CONF_ATOL


def test_draft_step_with_bad_anchors():
    # The fused call: bad requests draft -1, get NaN confidences, and the
    # schedule takes their survivals as 0 (the oracle's clamp of NaN).
    _say("case draft_step bad anchors")
    wl, anchors, bad = _bad_anchor_workload(1)
    g = H.to_device(wl, DEV)
    tok, conf, surv, lengths, order, info = D.dspark_draft_step(
        g["W1"], g["W2"], g["base"], torch.from_numpy(anchors).to(DEV), g["h"], g["w_conf"],
        g["sps"], GREEDY, want_order=True, want_info=True)
    torch.cuda.synchronize()
    t, c, s = tok.cpu().numpy(), conf.cpu().numpy(), surv.cpu().numpy()
    assert np.all(t[bad] == -1) and np.all(np.isnan(c[bad])) and np.all(np.isnan(s[bad]))
    H.check_schedule(s, wl["sps"], lengths.cpu().numpy(), order.cpu().numpy(), D.schedule_info(info))
    assert np.all(lengths.cpu().numpy()[bad] == 0)
