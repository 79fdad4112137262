"""Helpers for the GPU parity tests: move seeded workloads to the device and
compare the HIP path with the CPU oracle to the stated tolerances.

Tolerances (the oracle computes in fp64 unless the method fixes fp32):
  * draft tokens: exact wherever the oracle's top-1 / top-2 margin exceeds 1e-2
    on the forced sequence (the oracle replays each request with the GPU's
    previous tokens); elsewhere the GPU token must score within 1e-2 of the max;
  * Markov bias: |b_gpu - b_ref| <= 1e-3 * max(|b_ref|, rms of the b_ref row);
  * confidences: within 1e-4 absolute (on the forced sequence);
  * survival, sort order, lengths, B*, tau and Theta: bit-exact given the same
    confidences / survivals.
"""
from __future__ import annotations

import numpy as np
import torch

import draft_head_step_amd as D
from oracle import dspark_oracle as O

MARGIN = 1e-2
BIAS_RTOL = 1e-3
CONF_ATOL = 1e-4


def dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_device(wl: dict, device="cuda:0") -> dict:
    g = {}
    for k in ("W1", "W2", "h"):
        if wl.get(k) is not None:
            g[k] = dev_bf16(wl[k], device)
    for k in ("base", "uniforms", "w_conf", "sts", "sps", "conf"):
        if wl.get(k) is not None:
            g[k] = torch.from_numpy(np.ascontiguousarray(wl[k])).to(device)
    if wl.get("anchors") is not None:
        g["anchors"] = torch.from_numpy(wl["anchors"]).to(device)
    return g


def run_draft(wl, g, bias=False, layout=D.LAYOUT_RGV):
    """Run the draft on the device copies in g; `layout` picks the storage order of
    base / uniforms / bias_out (tiled copies are made here from the logical arrays)."""
    from draft_head_step_amd.inputs import from_tiled, to_tiled
    R, gm, V = wl["base"].shape
    dev = g["W1"].device
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(dev)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(dev)
    else:
        base, unif = g["base"], g.get("uniforms")
    bias_out = torch.full(base.shape, float("nan"), dtype=torch.float32, device=dev) if bias else None
    tok = D.dspark_markov_draft(g["W1"], g["W2"], base, g["anchors"], wl["mode"],
                                wl["temperature"], unif, bias_out=bias_out, layout=layout)
    torch.cuda.synchronize()
    b = None
    if bias:
        b = bias_out.cpu().numpy()
        if layout == D.LAYOUT_TILED:
            b = from_tiled(b, V)
    return tok.cpu().numpy(), b


def check_draft(wl, gpu_tokens, rows=None, gpu_bias=None):
    """Forced-sequence comparison of tokens (and optionally bias) on `rows`."""
    R, gm, V = wl["base"].shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    n_clear = n_amb = 0
    for k in range(gm):
        prev = wl["anchors"][rows] if k == 0 else gpu_tokens[rows, k - 1]
        u = None if wl["uniforms"] is None else wl["uniforms"][rows, k]
        x, s, margin = O.step_scores(wl["W1"], wl["W2"], wl["base"][rows, k], prev, wl["mode"],
                                     wl["temperature"], u)
        gt = gpu_tokens[rows, k]
        assert np.all((gt >= 0) & (gt < V)), "token id out of range"
        clear = margin > MARGIN
        bad = clear & (gt != x)
        assert not bad.any(), (f"step {k}: {bad.sum()} tokens differ where the margin exceeds "
                               f"{MARGIN}; rows {rows[bad][:8]}, gpu {gt[bad][:8]}, oracle {x[bad][:8]}")
        smax = s.max(axis=1)
        sg = s[np.arange(len(rows)), gt]
        assert np.all(smax - sg <= MARGIN), f"step {k}: a GPU token scores more than {MARGIN} below the max"
        n_clear += int(clear.sum())
        n_amb += int((~clear).sum())
        if gpu_bias is not None:
            ref = O.markov_bias(wl["W1"], wl["W2"], prev)
            got = gpu_bias[rows, k].astype(np.float64)
            rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
            tol = BIAS_RTOL * np.maximum(np.abs(ref), rms)
            err = np.abs(got - ref)
            assert np.all(err <= tol), f"step {k}: bias error {float((err / tol).max()):.3g} x tolerance"
    return n_clear, n_amb


def run_confidence(wl, g, gpu_tokens_dev):
    conf, surv = D.dspark_confidence(g["h"], g["W1"], g["anchors"], gpu_tokens_dev, g["w_conf"],
                                     g.get("sts"))
    torch.cuda.synchronize()
    return conf.cpu().numpy(), surv.cpu().numpy()


def check_confidence(wl, gpu_tokens, conf, surv):
    ref = O.confidence(wl["h"], wl["W1"], wl["anchors"], gpu_tokens, wl["w_conf"], wl["sts"])
    err = np.abs(conf.astype(np.float64) - ref)
    assert err.max() <= CONF_ATOL, f"confidence error {err.max():.3g}"
    # survival is bit-exact given the GPU's confidences
    assert np.array_equal(surv, O.survival(conf)), "survival differs from the fp32 running product"


def run_schedule(g_surv, g_sps):
    lengths, order, info = D.dspark_schedule(g_surv, g_sps, want_order=True, want_info=True)
    torch.cuda.synchronize()
    return lengths.cpu().numpy(), order.cpu().numpy(), D.schedule_info(info)


def check_schedule(surv_np, sps_np, lengths, order, info):
    ref = O.schedule(surv_np, sps_np)
    assert np.array_equal(order, ref["order"]), "sort order differs"
    assert np.array_equal(lengths, ref["lengths"]), "lengths differ"
    assert info.m_star == ref["m_star"] and info.B_star == ref["B_star"]
    assert info.tau_fx == ref["tau_fx"]
    assert info.tau == ref["tau"] and info.theta == ref["theta"]
    return ref


def check_rnn_draft(wl, hd, gpu_tokens, rows=None):
    """Forced-sequence comparison of RNN-head draft tokens on `rows`: the oracle
    replays each request with the GPU's previous tokens (its state evolving from
    them); where the oracle's margin exceeds MARGIN the ids must match, elsewhere
    the GPU's token must score within MARGIN of the maximum."""
    R, gm, V = wl["base"].shape
    rows = np.arange(R) if rows is None else np.asarray(rows)
    ref = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                      wl["mode"], wl["temperature"], wl["uniforms"], prev_tokens=gpu_tokens,
                      rows=rows, keep_scores=True)
    gt = gpu_tokens[rows]
    assert np.all((gt >= 0) & (gt < V)), "token id out of range"
    clear = ref["margin"] > MARGIN
    bad = clear & (gt != ref["tokens"])
    assert not bad.any(), (f"{bad.sum()} RNN tokens differ where the margin exceeds {MARGIN}; "
                           f"first at {np.argwhere(bad)[:4].tolist()}")
    sc = ref["scores"]
    smax = sc.max(axis=2)
    sg = np.take_along_axis(sc, gt[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    assert np.all(smax - sg <= MARGIN), "an RNN token scores more than the margin below the max"
    return int(clear.sum()), int((~clear).sum())


def check_rnn_state(gpu_state: np.ndarray, ref_state: np.ndarray, U_bits: np.ndarray,
                    W1_bits: np.ndarray) -> None:
    """The RNN head's last state (fp32 on the GPU) against the fp64 oracle on the
    forced sequence.

    Both round the state to bf16 where it enters a product, so they differ
    beyond the fp32 rounding of the update only where an element's fp32 and
    fp64 values fall on the two sides of a bf16 rounding boundary.  The state
    is a convex mix of the previous state and e + tanh(.), so |s| < S =
    1 + max|W1| (s_0 = 0); such an element enters the next product one bf16
    step apart, at most 2^(ceil(log2 S) - 8), which moves a pre-activation by
    at most max|U| times that, and the new state by at most (1 + S / 2) times
    the move (tanh slope <= 1; sigmoid slope <= 1/4 times |candidate - old|
    <= 2 S).  Every element must lie within two such flips (floor 1e-4), and
    the median error within 1e-6 (the bulk of the state matches to fp32
    rounding: a flip is rare)."""
    err = np.abs(gpu_state.astype(np.float64) - ref_state)
    S = 1.0 + float(np.abs(O.bf16_to_f64(W1_bits)).max())
    step = 2.0 ** (np.ceil(np.log2(S)) - 8)
    umax = float(np.abs(O.bf16_to_f64(U_bits)).max())
    tol = max(1e-4, 2 * umax * step * (1 + S / 2))
    assert err.max() <= tol, f"state error {err.max():.3g} above the two-flip bound {tol:.3g}"
    assert np.median(err) <= 1e-6, f"median state error {np.median(err):.3g}"
