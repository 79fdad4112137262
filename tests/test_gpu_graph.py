"""The fused draft step, the RNN-head draft and the acceptance probability
captured in a HIP graph.

The calls enqueue kernels only (no host synchronisation, no allocation, no
memset nodes: every clear is a kernel), so a captured call can be replayed.
Each replay runs after eager work that overwrites every output with garbage
and fills the workspace with 0xff; every replay must reproduce the eager
call's outputs bit for bit.
"""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

sys.path.insert(0, os.path.dirname(__file__))
import gpu_helpers as H  # noqa: E402

import draft_head_step_amd as D  # noqa: E402
from draft_head_step_amd.inputs import GREEDY, SAMPLE, Config, make_rnn_head, make_workload, to_tiled  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def _say(msg):
    print(msg, flush=True)


def _inputs(wl, g, layout):
    if layout == D.LAYOUT_TILED:
        base = torch.from_numpy(to_tiled(wl["base"])).to(DEV)
        unif = None if wl["uniforms"] is None else torch.from_numpy(to_tiled(wl["uniforms"])).to(DEV)
        return base, unif
    return g["base"], g.get("uniforms")


def _replay_and_compare(call, outs, ws):
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(REPLAYS):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5 + rep)
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"


CASES = [
    # name, R, gamma, V, r, d, mode
    ("ksplit", 70, 4, 3000, 512, 64, SAMPLE),
    ("plain", 300, 3, 5000, 256, 128, GREEDY),
    ("global", 2100, 4, 2000, 64, 32, GREEDY),   # 8400 candidates: the schedule's global path
]


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("name,R,g,V,r,d,mode", CASES)
def test_draft_step_replays_in_a_graph(name, R, g, V, r, d, mode, layout):
    _say(f"case graph draft_step {name} R={R} g={g} V={V} r={r} d={d} layout={layout}")
    cfg = Config("graph", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=0.9, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, sts=tuple(1.0 + 0.1 * k for k in range(g)),
                 seed=900 + R)
    wl = make_workload(cfg)
    gd = H.to_device(wl, DEV)
    base, unif = _inputs(wl, gd, layout)
    outs = [torch.empty((R, g), dtype=torch.int32, device=DEV),
            torch.empty((R, g), dtype=torch.float32, device=DEV),
            torch.empty((R, g), dtype=torch.float32, device=DEV),
            torch.empty((R,), dtype=torch.int32, device=DEV),
            torch.empty((R * g,), dtype=torch.int32, device=DEV),
            torch.empty((32,), dtype=torch.uint8, device=DEV)]
    ws = torch.empty(D.dspark_draft_step_workspace(R, g, V, r), dtype=torch.uint8, device=DEV)

    def call():
        D.dspark_draft_step(gd["W1"], gd["W2"], base, gd["anchors"], gd["h"], gd["w_conf"],
                            gd["sps"], mode, wl["temperature"], unif, sts_temp=gd.get("sts"),
                            tokens=outs[0], conf=outs[1], surv=outs[2], lengths=outs[3],
                            order=outs[4], info=outs[5], workspace=ws, layout=layout)

    _replay_and_compare(call, outs, ws)
    # and the replayed result is the oracle's (tokens on the forced sequence)
    H.check_draft(wl, outs[0].cpu().numpy(), None if R <= 300 else np.arange(0, R, 97))


@pytest.mark.parametrize("r,mode", [(64, GREEDY), (512, SAMPLE)])
def test_rnn_draft_replays_in_a_graph(r, mode):
    _say(f"case graph rnn r={r} mode={mode}")
    cfg = Config("graph", R=70, gamma=3, V=3000, r=r, d=1000, mode=mode, temperature=0.9,
                 w_std=0.2, base_std=1.0, seed=77)
    wl = make_workload(cfg)
    hd = make_rnn_head(cfg)
    gd = H.to_device(wl, DEV)
    U = H.dev_bf16(hd["U"], DEV)
    b = torch.from_numpy(hd["b"]).to(DEV)
    R, g = wl["R"], wl["gamma"]
    outs = [torch.empty((R, g), dtype=torch.int32, device=DEV),
            torch.empty((R, r), dtype=torch.float32, device=DEV)]
    ws = torch.empty(D.dspark_rnn_draft_workspace(R, g, wl["V"], r, wl["d"]), dtype=torch.uint8,
                     device=DEV)

    def call():
        D.dspark_rnn_draft(gd["W1"], gd["W2"], U, b, gd["base"], gd["h"], gd["anchors"], mode,
                           wl["temperature"], gd.get("uniforms"), tokens=outs[0],
                           state_out=outs[1], workspace=ws)

    _replay_and_compare(call, outs, ws)
    H.check_rnn_draft(wl, hd, outs[0].cpu().numpy())


@pytest.mark.parametrize("V", [70000, 4099])
def test_accept_prob_replays_in_a_graph(V):
    # 70000: the kernel that holds part of each row pair on chip (LDS attribute
    # set by the eager call before capture); 4099: the two-read kernel.
    _say(f"case graph accept_prob V={V}")
    from draft_head_step_amd.inputs import make_accept_workload
    from oracle import dspark_oracle as O
    wl = make_accept_workload(24, V, seed=V)
    d = torch.from_numpy(wl["draft"]).to(DEV)
    t = torch.from_numpy(wl["target"]).to(DEV)
    out = torch.empty((24,), dtype=torch.float32, device=DEV)
    scratch = torch.empty((16,), dtype=torch.uint8, device=DEV)   # no workspace: a stand-in

    def call():
        D.dspark_accept_prob(d, t, 0.9, out=out)

    _replay_and_compare(call, [out], scratch)
    ref = O.accept_prob(wl["draft"], wl["target"], 0.9)
    assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= 2e-5
