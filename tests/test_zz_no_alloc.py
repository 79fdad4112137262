"""The allocation-free draft entry point (static scratch) against the
workspace entry point, through the C ABI: two calls in a row, the second on a
smaller batch, in both layouts and both selection modes."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
sys.path.insert(0, os.path.dirname(__file__))

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import GREEDY, SAMPLE, Config, make_workload, to_tiled  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(wl, layout):
    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    conv = to_tiled if layout == D.LAYOUT_TILED else (lambda a: a)
    u = None if wl["uniforms"] is None else torch.from_numpy(conv(wl["uniforms"])).to(DEV)
    return (bf16(wl["W1"]), bf16(wl["W2"]), torch.from_numpy(conv(wl["base"])).to(DEV),
            torch.from_numpy(wl["anchors"]).to(DEV), u)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("mode,r", [(GREEDY, 128), (SAMPLE, 512)])
def test_noalloc_matches_workspace_entry(mode, r, layout):
    print(f"case noalloc mode={mode} r={r} layout={layout}", flush=True)
    big = make_workload(Config("na", R=300, gamma=4, V=6000, r=r, d=16, mode=mode,
                               temperature=0.9, w_std=0.2, base_std=1.0, seed=41))
    small = make_workload(Config("na", R=37, gamma=2, V=3001, r=r, d=16, mode=mode,
                                 temperature=1.1, w_std=0.2, base_std=1.0, seed=42))
    for wl in (big, small):   # the second call is smaller: no stale scratch may leak in
        W1, W2, base, anc, u = _dev(wl, layout)
        R, g = wl["R"], wl["gamma"]
        ref = D.dspark_markov_draft(W1, W2, base, anc, mode, wl["temperature"], u, layout=layout)
        got = torch.full((R, g), -7, dtype=torch.int32, device=DEV)
        D.dspark_markov_draft_noalloc(W1, W2, base, anc, got, mode, wl["temperature"], u,
                                      layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"R={R}: noalloc tokens differ from the workspace entry's"


def test_noalloc_rejects_above_its_limit():
    print("case noalloc limit", flush=True)
    W = torch.zeros((64, 16), dtype=torch.bfloat16, device=DEV)
    R, g = 4097, 8                      # R * gamma = 32776 > 32768
    anc = torch.zeros((R,), dtype=torch.int32, device=DEV)
    tok = torch.empty((R, g), dtype=torch.int32, device=DEV)
    with pytest.raises(D.DsparkError) as e:
        D.dspark_markov_draft_noalloc(W, W, None, anc, tok, GREEDY, gamma=g)
    assert e.value.status == 3
