"""GPU test of the W2 storage conversion (dspark_w2_store_from_rv): a row-by-row
[r, V] copy of W2 converts to the column-by-column [V, r] storage the draft
calls take, bit for bit (a pure data movement), at the benchmark shape and at
shapes with tails in both dimensions; a draft on the converted storage gives the
tokens of a draft on the original."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import CONFIGS, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("r,V", [(512, 129280), (256, 151936), (48, 1001), (1, 1), (70, 65),
                                 (64, 4096), (130, 63)])
def test_w2_store_from_rv_is_the_transpose(r, V):
    print(f"case w2 conversion r={r} V={V}", flush=True)
    rng = np.random.default_rng(r * 7 + V)
    rv = rng.integers(0, 1 << 16, size=(r, V), dtype=np.uint16)
    src = torch.from_numpy(rv.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = torch.full((V, r), float("nan"), dtype=torch.bfloat16, device=DEV)
    D.dspark_w2_store_from_rv(src, out=out)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, np.ascontiguousarray(rv.T))


def test_draft_on_converted_w2_matches():
    print("case w2 conversion then draft", flush=True)
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    rv = np.ascontiguousarray(wl["W2"].T)                  # [r, V], row by row
    src = H.dev_bf16(rv, DEV)
    w2 = D.dspark_w2_store_from_rv(src)
    t0 = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], D.GREEDY)
    t1 = D.dspark_markov_draft(g["W1"], w2, g["base"], g["anchors"], D.GREEDY)
    torch.cuda.synchronize()
    assert torch.equal(w2.view(torch.int16), g["W2"].view(torch.int16))
    assert torch.equal(t0, t1)
