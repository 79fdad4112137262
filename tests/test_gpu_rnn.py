"""GPU parity of the RNN-head draft (dspark_rnn_draft) against the CPU oracle's
reading of the RNN head, through the C ABI: tokens on the forced sequence
(the oracle's state follows the GPU's tokens), in both layouts, greedy and
sampling, every kernel variant the step uses (plain, K-split); its reduction
to the Markov head (bit-identical tokens); bad anchors."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import (CONFIGS, GREEDY, SAMPLE, Config, f32_to_bf16_bits,  # noqa: E402
                                         make_rnn_head, make_workload, to_tiled)
from oracle import dspark_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# The last state is compared by gpu_helpers.check_rnn_state (fp32 against fp64;
# bf16 roundings of the state that fall on different sides of a tie).


def _say(msg):
    print(msg, flush=True)


def _run(wl, hd, layout, anchors=None):
    g = H.to_device(wl, DEV)
    U = H.dev_bf16(hd["U"], DEV)
    b = torch.from_numpy(hd["b"]).to(DEV)
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(DEV)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(DEV)
    else:
        base, unif = g["base"], g.get("uniforms")
    anc = g["anchors"] if anchors is None else torch.from_numpy(anchors).to(DEV)
    R, r = wl["R"], wl["W1"].shape[1]
    state = torch.full((R, r), float("nan"), dtype=torch.float32, device=DEV)
    tok = D.dspark_rnn_draft(g["W1"], g["W2"], U, b, base, g["h"], anc, wl["mode"],
                             wl["temperature"], unif, state_out=state, layout=layout)
    torch.cuda.synchronize()
    _run.state = state.cpu().numpy()
    return tok.cpu().numpy(), g, base, unif


CASES = [
    # R, gamma, V, r, d, mode
    (4, 5, 4096, 64, 256, GREEDY),
    (33, 3, 1001, 48, 40, SAMPLE),
    (70, 4, 3000, 256, 104, SAMPLE),
    (40, 3, 5000, 512, 64, SAMPLE),      # rank 512 sampling: K-split pairs on dense rows
    (300, 2, 3000, 512, 16, GREEDY),     # rank 512 greedy: eight plain waves, two staging rounds
    (130, 2, 999, 128, 32, GREEDY),
    (70, 3, 3000, 64, 1000, GREEDY),     # pre-activation GEMM: K in 4 splits, ragged K and M tails
    (33, 3, 1001, 48, 520, SAMPLE),      # 2 splits, 96 units in a 128-unit tile
    (1, 1, 100, 16, 8, GREEDY),          # the smallest shapes: one request, one step, r = 16, d = 8
    (17, 1, 2000, 32, 24, SAMPLE),       # one step; 16 + 1 requests (a one-request state tile)
]


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("R,g,V,r,d,mode", CASES)
def test_rnn_draft_matches_oracle(R, g, V, r, d, mode, layout):
    _say(f"case rnn R={R} g={g} V={V} r={r} d={d} mode={mode} layout={layout}")
    cfg = Config("rnn", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=0.9, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, seed=600 + R)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    toks, _, _, _ = _run(wl, hd, layout)
    n_clear, n_amb = H.check_rnn_draft(wl, hd, toks)
    assert n_clear > 0
    # the last state itself, on the forced sequence (fp32 state against fp64)
    ref = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                      wl["mode"], wl["temperature"], wl["uniforms"], prev_tokens=toks,
                      keep_state=True)
    H.check_rnn_state(_run.state, ref["states"][:, -1, :], hd["U"], wl["W1"])


def test_rnn_draft_dsv4_shape():
    # R = 256, gamma = 5, V = 129280, r = 512, d = 7168, sampling; every
    # 32-request tile sampled.
    _say("case rnn dsv4 shape")
    cfg = CONFIGS["dsv4"]
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    toks, _, _, _ = _run(wl, hd, D.LAYOUT_RGV)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 255], [t + rng.integers(32) for t in range(0, 256, 32)]]))
    H.check_rnn_draft(wl, hd, toks, rows)
    ref = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                      wl["mode"], wl["temperature"], wl["uniforms"], prev_tokens=toks, rows=rows,
                      keep_state=True)
    H.check_rnn_state(_run.state[rows], ref["states"][:, -1, :], hd["U"], wl["W1"])


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("r,mode", [(64, GREEDY), (512, SAMPLE), (512, GREEDY)])
def test_saturated_gate_drafts_the_markov_tokens(r, mode, layout):
    # Gate bias +100 (g = 1 in fp32), no candidate correction: the state is the
    # embedding row, so the RNN draft must equal the Markov draft bit for bit.
    _say(f"case rnn = markov r={r} mode={mode} layout={layout}")
    cfg = Config("rnn", R=70, gamma=4, V=3000, r=r, d=32, mode=mode, temperature=0.8, w_std=0.2,
                 base_std=1.0, seed=17)
    wl = make_workload(cfg)
    rng = np.random.default_rng(3)
    U = np.zeros((2 * r, 2 * r + 32), np.float32)
    U[:r] = rng.uniform(-0.05, 0.05, size=(r, 2 * r + 32))
    hd = {"U": f32_to_bf16_bits(U),
          "b": np.concatenate([np.full(r, 100.0), np.zeros(r)]).astype(np.float32)}
    toks, g, base, unif = _run(wl, hd, layout)
    ref = D.dspark_markov_draft(g["W1"], g["W2"], base, g["anchors"], mode, wl["temperature"],
                                unif, layout=layout).cpu().numpy()
    assert np.array_equal(toks, ref)


def test_rnn_bad_anchors_give_minus_one():
    _say("case rnn bad anchors")
    cfg = Config("rnn", R=40, gamma=3, V=2000, r=64, d=16, w_std=0.2, base_std=1.0, seed=19)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    anchors = wl["anchors"].copy()
    bad = np.array([1, 7, 39])
    anchors[bad] = np.array([-5, 2000, 1 << 29], np.int32)
    toks, _, _, _ = _run(wl, hd, D.LAYOUT_RGV, anchors)
    good, _, _, _ = _run(wl, hd, D.LAYOUT_RGV)
    assert np.all(toks[bad] == -1)
    keep = np.setdiff1d(np.arange(40), bad)
    assert np.array_equal(toks[keep], good[keep])
