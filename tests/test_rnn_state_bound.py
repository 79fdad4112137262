"""The RNN head's last-state tolerance (gpu_helpers.check_rnn_state) against an
fp32 run of the same recurrence on the CPU (CPU only).

The GPU keeps the state in fp32; the oracle in fp64; both round it to bf16
where it enters a product.  An fp32 numpy run of the oracle's recurrence (same
bf16 operands, same forced tokens) differs from the fp64 oracle by the same
mechanism the tolerance is derived from: fp32 rounding of each update, and now
and then a state element whose fp32 and fp64 values round to different bf16
neighbours.  Its last state must pass the same check the GPU's state passes.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

from draft_head_step_amd.inputs import GREEDY, SAMPLE, Config, make_rnn_head, make_workload  # noqa: E402
from oracle import dspark_oracle as O  # noqa: E402


def _update32(s_prev, e, h_k, U, b):
    r = e.shape[1]
    Uf = O.bf16_to_f64(U).astype(np.float32)
    u = np.concatenate([O.bf16_round(s_prev).astype(np.float32), e.astype(np.float32),
                        h_k.astype(np.float32)], axis=1)
    pre = u @ Uf.T + np.asarray(b, dtype=np.float32)[None, :]
    g = np.float32(1.0) / (np.float32(1.0) + np.exp(-pre[:, :r]))
    cand = e.astype(np.float32) + np.tanh(pre[:, r:])
    return (g * cand + (np.float32(1.0) - g) * s_prev).astype(np.float32)


@pytest.mark.parametrize("R,g,V,r,d,mode", [(257, 5, 257, 496, 464, SAMPLE),
                                            (257, 3, 1000, 368, 832, GREEDY),
                                            (64, 6, 500, 304, 1256, GREEDY)])
def test_fp32_recurrence_passes_the_state_check(R, g, V, r, d, mode):
    cfg = Config("bound", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=1.3, w_std=0.2,
                 base_std=1.0, seed=40 + r)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    ref = O.rnn_draft(wl["W1"], wl["W2"], hd["U"], hd["b"], wl["base"], wl["h"], wl["anchors"],
                      mode, cfg.temperature, wl["uniforms"], keep_state=True)
    toks = ref["tokens"]
    s = np.zeros((R, r), np.float32)
    prev = wl["anchors"].astype(np.int64)
    for k in range(g):
        s = _update32(s, O.bf16_to_f64(wl["W1"][prev]), O.bf16_to_f64(wl["h"][:, k, :]),
                      hd["U"], hd["b"])
        prev = toks[:, k].astype(np.int64)
    err = np.abs(s.astype(np.float64) - ref["states"][:, -1, :])
    assert err.max() > 0.0          # the two runs do differ
    H.check_rnn_state(s, ref["states"][:, -1, :], hd["U"], wl["W1"])
