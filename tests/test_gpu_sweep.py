"""Seeded sweeps over shapes drawn at random (requests, positions, vocabulary
sizes that are and are not multiples of the 32-entry chunk, every Markov rank
class, hidden sizes, greedy and sampling at several temperatures, both logits
layouts, with and without STS):
  * the fused draft step, compared with the CPU oracle to the bars stated in
    gpu_helpers, and its tokens with those of dspark_markov_draft on the same
    inputs;
  * the RNN-head draft, tokens on the forced sequence and the last state;
  * the verification side (flattening and greedy accept / correct bit-exact,
    the acceptance probability within 2e-5 as in test_gpu_verify);
  * the acceptance probability alone at vocabularies up to 200000, across the
    parts of a row pair its holding kernel keeps on chip.

The draw is fixed (numpy seed), so a failing case can be re-run by its id.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import GREEDY, SAMPLE, Config, make_workload, to_tiled  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 3, 31, 32, 33, 64, 97, 130, 257, 300]))
        g = int(rng.integers(1, 10))
        V = int(rng.choice([7, 33, 257, 1000, 2048, 3001, 4096]))
        r = int(16 * rng.integers(1, 33))                  # 16 .. 512
        d = int(4 * rng.integers(1, 300))                  # multiples of 4
        mode = int(rng.choice([GREEDY, SAMPLE]))
        temp = float(rng.choice([0.5, 1.0, 1.7]))
        sts = bool(rng.integers(0, 2))
        layout = int(rng.choice([D.LAYOUT_RGV, D.LAYOUT_TILED]))
        out.append((i, R, g, V, r, d, mode, temp, sts, layout))
    return out


CASES = _cases()


@pytest.mark.parametrize("i,R,g,V,r,d,mode,temp,sts,layout", CASES,
                         ids=[f"sweep{c[0]}" for c in CASES])
def test_fused_step_sweep(i, R, g, V, r, d, mode, temp, sts, layout):
    print(f"case sweep{i}: R={R} g={g} V={V} r={r} d={d} mode={mode} T={temp} sts={sts} "
          f"layout={layout}", flush=True)
    cfg = Config(f"sweep{i}", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=temp,
                 w_std=0.2, base_std=1.0, wconf_std=0.05,
                 sts=tuple(1.0 + 0.15 * k for k in range(g)) if sts else None, seed=900 + i)
    wl = make_workload(cfg)
    dev = H.to_device(wl, DEV)
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(DEV)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(DEV)
    else:
        base, unif = dev["base"], dev.get("uniforms")
    tok, conf, surv, lengths, order, info = D.dspark_draft_step(
        dev["W1"], dev["W2"], base, dev["anchors"], dev["h"], dev["w_conf"], dev["sps"], mode,
        temp, unif, sts_temp=dev.get("sts"), want_order=True, want_info=True, layout=layout)
    ref_tok = D.dspark_markov_draft(dev["W1"], dev["W2"], base, dev["anchors"], mode, temp, unif,
                                    layout=layout)
    torch.cuda.synchronize()
    toks = tok.cpu().numpy()
    assert np.array_equal(toks, ref_tok.cpu().numpy()), "fused tokens differ from dspark_markov_draft"
    H.check_draft(wl, toks)
    H.check_confidence(wl, toks, conf.cpu().numpy(), surv.cpu().numpy())
    H.check_schedule(surv.cpu().numpy(), wl["sps"], lengths.cpu().numpy(), order.cpu().numpy(),
                     D.schedule_info(info))


# ---------------------------------------------------------------- RNN head
def _rnn_cases(n=24, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 17, 32, 33, 64, 100, 130, 257]))
        g = int(rng.integers(1, 7))
        V = int(rng.choice([33, 257, 1000, 3001]))
        r = int(16 * rng.integers(1, 33))
        d = int(8 * rng.integers(1, 160))                  # multiples of 8 (the RNN head's bound)
        mode = int(rng.choice([GREEDY, SAMPLE]))
        temp = float(rng.choice([0.7, 1.0, 1.3]))
        layout = int(rng.choice([D.LAYOUT_RGV, D.LAYOUT_TILED]))
        out.append((i, R, g, V, r, d, mode, temp, layout))
    return out


RNN_CASES = _rnn_cases()


@pytest.mark.parametrize("i,R,g,V,r,d,mode,temp,layout", RNN_CASES,
                         ids=[f"rnn{c[0]}" for c in RNN_CASES])
def test_rnn_draft_sweep(i, R, g, V, r, d, mode, temp, layout):
    print(f"case rnn sweep{i}: R={R} g={g} V={V} r={r} d={d} mode={mode} T={temp} "
          f"layout={layout}", flush=True)
    from draft_head_step_amd.inputs import make_rnn_head
    from oracle import dspark_oracle as O
    cfg = Config(f"rnn{i}", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=temp, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, seed=1300 + i)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    dev = H.to_device(wl, DEV)
    U = H.dev_bf16(hd["U"], DEV)
    b = torch.from_numpy(hd["b"]).to(DEV)
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(DEV)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(DEV)
    else:
        base, unif = dev["base"], dev.get("uniforms")
    state = torch.full((R, r), float("nan"), dtype=torch.float32, device=DEV)
    tok = D.dspark_rnn_draft(dev["W1"], dev["W2"], U, b, base, dev["h"], dev["anchors"], mode, temp,
                             unif, state_out=state, layout=layout)
    torch.cuda.synchronize()
    toks = tok.cpu().numpy()
    H.check_rnn_draft(wl, hd, toks)
    ref = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                      mode, temp, wl["uniforms"], prev_tokens=toks, keep_state=True)
    H.check_rnn_state(state.cpu().numpy(), ref["states"][:, -1, :], hd["U"], wl["W1"])


# ---------------------------------------------------------------- verification side
def _verify_cases(n=16, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 63, 64, 65, 500, 1025, 2000]))
        g = int(rng.integers(1, 12))
        V = int(rng.choice([2, 37, 1000, 4097, 30000]))
        rate = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
        T = float(rng.choice([0.6, 1.0, 1.4]))
        while R * (1 + g) * V > 40_000_000:      # keep the target logits near 160 MB at most
            V = max(2, V // 4)
        out.append((i, R, g, V, rate, T))
    return out


VERIFY_CASES = _verify_cases()


@pytest.mark.parametrize("i,R,g,V,rate,T", VERIFY_CASES, ids=[f"verify{c[0]}" for c in VERIFY_CASES])
def test_verify_sweep(i, R, g, V, rate, T):
    print(f"case verify sweep{i}: R={R} g={g} V={V} rate={rate} T={T}", flush=True)
    from draft_head_step_amd.inputs import make_accept_workload, make_verify_workload
    from oracle import dspark_oracle as O

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    wl = make_verify_workload(R, g, V, seed=1700 + i, match_rate=rate)
    ref = O.verify_pack(wl["anchors"], wl["tokens"], wl["lengths"], wl["pos0"])
    ft, fp, fr, cu = D.dspark_verify_pack(dev(wl["anchors"]), dev(wl["tokens"]),
                                          dev(wl["lengths"]), dev(wl["pos0"]))
    torch.cuda.synchronize()
    B = ref["B"]
    assert np.array_equal(cu.cpu().numpy(), ref["cu_seqlens"])
    assert np.array_equal(ft.cpu().numpy()[:B], ref["tokens"])
    assert np.array_equal(fp.cpu().numpy()[:B], ref["positions"])
    assert np.array_equal(fr.cpu().numpy()[:B], ref["request"])
    # greedy accept / correct on the flattened target rows
    tl = np.ascontiguousarray(np.concatenate(
        [wl["target"][r, :ref["cu_seqlens"][r + 1] - ref["cu_seqlens"][r]] for r in range(R)], axis=0))
    rg = O.verify_greedy(tl, ref["cu_seqlens"], wl["tokens"], wl["lengths"])
    acc, nxt, amax = D.dspark_verify_greedy(dev(tl), dev(ref["cu_seqlens"]), dev(wl["tokens"]))
    torch.cuda.synchronize()
    assert np.array_equal(amax.cpu().numpy()[:B], rg["target_argmax"])
    assert np.array_equal(acc.cpu().numpy(), rg["accepted"])
    assert np.array_equal(nxt.cpu().numpy(), rg["next_token"])
    # acceptance probability on a few row pairs of this vocabulary
    aw = make_accept_workload(min(B, 16), V, seed=1800 + i)
    ra = O.accept_prob(aw["draft"], aw["target"], T)
    ga = D.dspark_accept_prob(dev(aw["draft"]), dev(aw["target"]), T).cpu().numpy()
    assert np.abs(ga.astype(np.float64) - ra).max() <= 2e-5


def _accept_cases(n_cases=12, seed=2024):
    # V up to 200000, so the row pairs cross the parts the holding kernel keeps
    # in registers (49152 entries) and LDS (65536) and stream the rest; about
    # one V in four is not a multiple of four (the two-read kernel).
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        V = int(rng.integers(2, 200_001))
        if rng.random() < 0.75:
            V = max(4, V // 4 * 4)
        n = int(rng.integers(1, 13))
        T = float(rng.choice([0.5, 0.8, 1.0, 1.7]))
        out.append((i, n, V, T))
    return out


ACCEPT_CASES = _accept_cases()


@pytest.mark.parametrize("i,n,V,T", ACCEPT_CASES, ids=[f"accept{c[0]}" for c in ACCEPT_CASES])
def test_accept_prob_sweep(i, n, V, T):
    print(f"case accept sweep{i}: n={n} V={V} T={T}", flush=True)
    from draft_head_step_amd.inputs import make_accept_workload
    from oracle import dspark_oracle as O
    aw = make_accept_workload(n, V, seed=1900 + i)
    ra = O.accept_prob(aw["draft"], aw["target"], T)
    ga = D.dspark_accept_prob(torch.from_numpy(aw["draft"]).to(DEV),
                              torch.from_numpy(aw["target"]).to(DEV), T).cpu().numpy()
    assert np.abs(ga.astype(np.float64) - ra).max() <= 2e-5
