"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances are stated in gpu_helpers.  Every workload is seeded; the large ones
use the full sizes of the benchmarked configurations, with the draft checked on
sampled requests (the oracle recomputes those requests' steps one by one on
the GPU's token sequence).
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
from draft_head_step_amd.inputs import CONFIGS, GREEDY, SAMPLE, Config, make_workload  # noqa: E402
from oracle import dspark_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _full_path_check(wl, rows=None, bias_rows=True, layout=D.LAYOUT_RGV):
    g = H.to_device(wl, DEV)
    toks, bias = H.run_draft(wl, g, bias=bias_rows, layout=layout)
    n_clear, n_amb = H.check_draft(wl, toks, rows, bias)
    tok_dev = torch.from_numpy(toks).to(DEV)
    conf, surv = H.run_confidence(wl, g, tok_dev)
    H.check_confidence(wl, toks, conf, surv)
    lengths, order, info = H.run_schedule(torch.from_numpy(surv).to(DEV), g["sps"])
    H.check_schedule(surv, wl["sps"], lengths, order, info)
    return toks, n_clear, n_amb


# --------------------------------------------------------------------------- tiny

@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_tiny_greedy_end_to_end(layout):
    _say(f"case tiny greedy layout={layout}")
    wl = make_workload(CONFIGS["tiny"])
    _, n_clear, _ = _full_path_check(wl, layout=layout)
    assert n_clear > 0


def test_tiny_bias_dominant_moves_tokens():
    _say("case tiny bias-dominant")
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    toks, _, _ = _full_path_check(wl)
    assert (toks != np.argmax(wl["base"], axis=2)).any()


@pytest.mark.parametrize("T,layout", [(1.0, D.LAYOUT_RGV), (0.7, D.LAYOUT_RGV), (0.7, D.LAYOUT_TILED)])
def test_tiny_sampling(T, layout):
    _say(f"case tiny sample T={T} layout={layout}")
    cfg = dataclasses.replace(CONFIGS["tiny"], mode=SAMPLE, temperature=T)
    wl = make_workload(cfg, w_std=0.2)
    _full_path_check(wl, layout=layout)


def test_deterministic_repeat():
    _say("case determinism")
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    a, ba = H.run_draft(wl, g, bias=True)
    b, bb = H.run_draft(wl, g, bias=True)
    assert np.array_equal(a, b) and np.array_equal(ba.view(np.uint32), bb.view(np.uint32))


def test_concurrent_host_threads_on_separate_streams():
    # Two host threads, each with its own stream, outputs and workspace (the
    # documented condition for concurrent calls), draft the same batch: every
    # result equals the single-threaded one.
    _say("case concurrent host threads")
    import threading
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    ref = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], GREEDY).cpu().numpy()
    results, errors = [], []

    def worker():
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(5):
                    t = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], GREEDY,
                                              stream=st)
                    st.synchronize()
                    results.append(t.cpu().numpy())
        except Exception as exc:  # noqa: BLE001
            errors.append(exc)

    th = [threading.Thread(target=worker) for _ in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    assert len(results) == 10 and all(np.array_equal(r, ref) for r in results)


def test_workspace_contents_do_not_matter():
    # The call clears the words it combines into: a workspace full of 0xff, and
    # the same workspace again after a call on other inputs, give the same tokens.
    _say("case dirty workspace")
    cfg = dataclasses.replace(CONFIGS["tiny"], mode=SAMPLE, temperature=0.8)
    wl = make_workload(cfg, w_std=0.3)
    g = H.to_device(wl, DEV)
    R, gm, V = wl["base"].shape
    need = D.dspark_markov_draft_workspace(R, gm, V, wl["r"])
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    args = (g["W1"], g["W2"], g["base"], g["anchors"], SAMPLE, 0.8, g["uniforms"])
    a = D.dspark_markov_draft(*args, workspace=ws).cpu().numpy()
    other = torch.flip(g["anchors"], [0]).contiguous()
    D.dspark_markov_draft(g["W1"], g["W2"], g["base"], other, SAMPLE, 0.8, g["uniforms"],
                          workspace=ws)
    b = D.dspark_markov_draft(*args, workspace=ws).cpu().numpy()
    assert np.array_equal(a, b)
    H.check_draft(wl, a)


# --------------------------------------------------------------------------- edges

EDGE = [
    # R, gamma, V, r, d, mode
    (1, 1, 2, 16, 8, GREEDY),
    (33, 3, 1001, 48, 40, SAMPLE),      # V % 4 != 0 (scalar epilogue), r below its bucket
    (5, 2, 4099, 128, 24, GREEDY),
    (70, 4, 3000, 256, 100, SAMPLE),    # partial R blocks, d % 8 != 0
    (3, 6, 64, 512, 16, GREEDY),        # V smaller than a chunk group, r = 512
    (300, 2, 777, 64, 64, GREEDY),      # two 256-request blocks, last one partial
    (40, 3, 1001, 512, 16, SAMPLE),     # rank 512 (K-split) with the scalar epilogue
    (40, 3, 1001, 512, 16, GREEDY),     # rank 512 (plain, direct-to-LDS W2), scalar epilogue
    (130, 2, 999, 256, 16, GREEDY),     # rank 256, 4-wave blocks, scalar epilogue
    (300, 2, 3000, 512, 16, GREEDY),    # rank 512, 8 waves: W1 rows staged in two rounds
]


@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("R,g,V,r,d,mode", EDGE)
def test_edge_shapes(R, g, V, r, d, mode, layout, bias):
    # With and without the bias output: the two select different kernel
    # instances (the hot path never writes the bias).
    _say(f"case edge R={R} g={g} V={V} r={r} d={d} mode={mode} layout={layout} bias={bias}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=r, d=d, mode=mode, temperature=0.9, w_std=0.2,
                 base_std=1.0, wconf_std=0.1, seed=100 + R)
    wl = make_workload(cfg)
    _full_path_check(wl, layout=layout, bias_rows=bias)


# Rank 512 without a bias output, in the layouts and request counts that pick
# each kernel the hot path runs: sampling -> K-split pairs (1, 2 or 4 pairs per
# workgroup: R <= 32, R <= 96, R > 96); greedy -> the plain kernel with 1, 2,
# 4 (deeper rings) or 8 waves.  V = 5000 has a partial last chunk, V = 8192 none.
RANK512 = [
    (20, 3, 5000, SAMPLE), (60, 3, 8192, SAMPLE), (100, 3, 8192, SAMPLE), (200, 2, 5000, SAMPLE),
    (20, 3, 8192, GREEDY), (40, 2, 5000, GREEDY), (100, 3, 5000, GREEDY),
    (300, 2, 8192, GREEDY),
]


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("R,g,V,mode", RANK512)
def test_rank512_without_bias_output(R, g, V, mode, layout):
    _say(f"case rank512 no-bias R={R} g={g} V={V} mode={mode} layout={layout}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=512, d=64, mode=mode, temperature=0.8, w_std=0.1,
                 base_std=1.0, wconf_std=0.1, seed=900 + R)
    _full_path_check(make_workload(cfg), layout=layout, bias_rows=False)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_largest_row_major_vocabulary(layout):
    # gamma * V just below 2^22, the row-major limit of 32-bit element offsets
    # per request block (the tiled layout takes the same V).
    V = (1 << 22) - 32
    _say(f"case V={V} layout={layout}")
    cfg = Config("edge", R=5, gamma=1, V=V, r=64, d=16, w_std=0.2, base_std=1.0, seed=31)
    wl = make_workload(cfg)
    _full_path_check(wl, layout=layout)


def test_tiled_layout_at_its_size_limit():
    # ceil(V/32) * R = 2^24 - 128: one step of the column-tiled logits is just below
    # 2^31 bytes, and the last 256-request block holds one row past R, which the
    # kernel sends out of range.  The logits (2 GiB) are drawn on the device; the
    # tokens are checked on sampled rows, the first and last included.
    from draft_head_step_amd.inputs import make_head
    R, V, g, r = (1 << 17) - 1, 4096, 1, 64
    _say(f"case tiled size limit R={R} V={V} r={r}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=r, d=16, mode=GREEDY, temperature=1.0, w_std=0.3,
                 base_std=1.0, wconf_std=0.1, seed=77)
    hd = make_head(cfg)
    gw = H.to_device({"W1": hd["W1"], "W2": hd["W2"], "anchors": hd["anchors"]}, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    C = (V + 31) // 32
    assert C * R < (1 << 24)
    tiled = torch.randn((g, C, 32, R), generator=gen, device=DEV)
    tok = D.dspark_markov_draft(gw["W1"], gw["W2"], tiled, gw["anchors"], GREEDY, 1.0, None,
                                layout=D.LAYOUT_TILED)
    torch.cuda.synchronize()
    rows = _sample_rows(R, 12, 5)
    sel = tiled.index_select(3, torch.from_numpy(rows).to(DEV))
    base_rows = sel.permute(3, 0, 1, 2).reshape(len(rows), g, C * 32)[:, :, :V].cpu().numpy()
    del tiled, sel
    wl = {"W1": hd["W1"], "W2": hd["W2"], "anchors": hd["anchors"][rows], "base": base_rows,
          "mode": GREEDY, "temperature": 1.0, "uniforms": None}
    H.check_draft(wl, tok.cpu().numpy()[rows])


@pytest.mark.parametrize("r,mode", [(64, GREEDY), (512, GREEDY), (512, SAMPLE)])
def test_unaligned_base_uses_scalar_path(r, mode):
    _say(f"case unaligned base r={r} mode={mode}")
    cfg = Config("edge", R=6, gamma=3, V=4096, r=r, d=32, w_std=0.2, mode=mode, seed=7)
    wl = make_workload(cfg)
    g = H.to_device(wl, DEV)
    R, gm, V = wl["base"].shape
    big = torch.empty(R * gm * V + 1, dtype=torch.float32, device=DEV)
    base = big[1:].view(R, gm, V)
    base.copy_(g["base"])
    tok = D.dspark_markov_draft(g["W1"], g["W2"], base, g["anchors"], mode, wl["temperature"],
                                g.get("uniforms"))
    toks = tok.cpu().numpy()
    H.check_draft(wl, toks)


def test_exact_ties_resolve_to_smallest_id():
    _say("case ties")
    R, gm, V, r = 40, 2, 5000, 64
    rng = np.random.default_rng(3)
    base = rng.uniform(-1, 1, size=(R, gm, V)).astype(np.float32)
    for m in range(R):
        for k in range(gm):
            ids = np.sort(rng.choice(V, size=4, replace=False))
            base[m, k, ids] = 7.5
    wl = {"W1": np.zeros((V, r), np.uint16), "W2": np.zeros((V, r), np.uint16), "base": base,
          "anchors": rng.integers(0, V, size=R).astype(np.int32), "mode": GREEDY,
          "temperature": 1.0, "uniforms": None}
    g = H.to_device(wl, DEV)
    toks, _ = H.run_draft(wl, g)
    want = np.argmax(base, axis=2)
    assert np.array_equal(toks, want)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_negative_maxima_and_zero_ties(layout):
    # Every logit negative, with exact ties at the maximum (-1.5 in the first
    # position, signed zeros in the second) spread over distant V groups: the
    # cross-group combine must order negative scores and treat -0 == +0.
    _say(f"case negative maxima layout={layout}")
    R, gm, V, r = 70, 2, 20000, 64
    rng = np.random.default_rng(11)
    base = rng.uniform(-10, -2, size=(R, gm, V)).astype(np.float32)
    for m in range(R):
        ids = np.sort(rng.choice(V, size=3, replace=False))
        base[m, 0, ids] = -1.5
        ids = np.sort(rng.choice(V, size=4, replace=False))
        base[m, 1, ids] = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)[rng.permutation(4)]
    wl = {"W1": np.zeros((V, r), np.uint16), "W2": np.zeros((V, r), np.uint16), "base": base,
          "anchors": rng.integers(0, V, size=R).astype(np.int32), "mode": GREEDY,
          "temperature": 1.0, "uniforms": None}
    g = H.to_device(wl, DEV)
    toks, _ = H.run_draft(wl, g, layout=layout)
    assert np.array_equal(toks, np.argmax(base, axis=2))


# --------------------------------------------------------------------------- scheduler

def _sched_case(c, sps):
    gs = torch.from_numpy(c).to(DEV)
    surv = D.dspark_survival(gs)
    torch.cuda.synchronize()
    s = surv.cpu().numpy()
    assert np.array_equal(s, O.survival(c))
    lengths, order, info = H.run_schedule(surv, torch.from_numpy(sps).to(DEV))
    return H.check_schedule(s, sps, lengths, order, info)


@pytest.mark.parametrize("R,g", [(1, 1), (4, 5), (1000, 2), (2048, 4), (2731, 3), (3277, 5),
                                 (5000, 7), (100003, 6)])
def test_schedule_sizes_and_paths(R, g):
    # 2048 x 4 = 8192 is the largest single-workgroup (LDS) case; 2731 x 3 = 8193 the
    # smallest tiled (workspace) case; 100003 x 6 has 586 tiles, more than a
    # scatter workgroup sums itself, so the digit bases come from a separate scan.
    _say(f"case schedule R={R} g={g}")
    rng = np.random.default_rng(R * 31 + g)
    c = rng.beta(6, 1.5, size=(R, g)).astype(np.float32)
    from draft_head_step_amd.inputs import sps_table
    _sched_case(c, sps_table("staircase", R * (1 + g)))


def test_schedule_ties_and_saturation():
    _say("case schedule ties")
    rng = np.random.default_rng(9)
    R, g = 2000, 6
    c = rng.choice(np.array([1.0, 0.5, 0.0, 0.75], np.float32), size=(R, g))
    B = np.arange(1, R * (1 + g) + 1)
    _sched_case(c, (0.999 ** (B / 64.0)).astype(np.float32))


@pytest.mark.parametrize("R,g", [(40, 5), (3000, 4)])
def test_schedule_signed_zero_sps_ties(R, g):
    # SPS entries of -0.0 and +0.0 alternate, so every Theta is a signed zero; they
    # compare equal, and the first argmax (m* = 0) must win on both paths.
    _say(f"case schedule signed-zero SPS R={R} g={g}")
    rng = np.random.default_rng(R)
    c = rng.uniform(0.2, 1.0, size=(R, g)).astype(np.float32)
    sps = np.zeros(R * (1 + g), np.float32)
    sps[R - 1::2] = np.float32(-0.0)
    assert O.schedule(O.survival(c), sps)["m_star"] == 0
    _sched_case(c, sps)


@pytest.mark.parametrize("K", [1, 100, 777])
def test_schedule_capacity_step_is_top_k(K):
    _say(f"case schedule top-K K={K}")
    rng = np.random.default_rng(K)
    R, g = 300, 5
    c = rng.uniform(0.05, 1, size=(R, g)).astype(np.float32)
    K = max(K, R)
    sps = (np.arange(1, R * (1 + g) + 1) <= K).astype(np.float32)
    ref = _sched_case(c, sps)
    assert ref["B_star"] == K


def test_schedule_at_the_candidate_limit():
    # R * gamma = DSPARK_MAX_CANDIDATES = 2^23: 8192 tiles on the tiled path.
    _say("case schedule at 2^23 candidates")
    R, g = 1 << 20, 8
    rng = np.random.default_rng(23)
    c = rng.uniform(0.05, 1.0, size=(R, g)).astype(np.float32)
    from draft_head_step_amd.inputs import sps_table
    _sched_case(c, sps_table("staircase", R * (1 + g)))


def test_sched_stress_workload():
    _say("case sched_stress")
    wl = make_workload(CONFIGS["sched_stress"])
    _sched_case(wl["conf"], wl["sps"])


def _sched_ex_case(a, sps, mode, K=0):
    gs = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    gsps = None if sps is None else torch.from_numpy(sps).to(DEV)
    lengths, order, info = D.dspark_schedule_ex(gs, gsps, mode=mode, capacity=K, want_order=True,
                                                want_info=True)
    torch.cuda.synchronize()
    ref = O.schedule_early_stop(a, sps) if mode == D.SCHED_EARLY_STOP else O.schedule_capacity(a, K)
    inf = D.schedule_info(info)
    assert np.array_equal(order.cpu().numpy(), ref["order"]), "sort order differs"
    assert np.array_equal(lengths.cpu().numpy(), ref["lengths"]), "lengths differ"
    assert inf.m_star == ref["m_star"] and inf.B_star == ref["B_star"]
    assert inf.tau_fx == ref["tau_fx"] and inf.tau == ref["tau"] and inf.theta == ref["theta"]
    return ref


@pytest.mark.parametrize("R,g,kind,slope", [(50, 5, "stair_lin", 0.002), (256, 7, "stair", 0.0),
                                            (1000, 8, "stair", 0.0), (1100, 8, "stair", 0.0),
                                            (1100, 8, "lin", 0.00004), (3000, 5, "lin", 0.00002),
                                            (3000, 5, "lin", 0.00005)])
def test_schedule_early_stop(R, g, kind, slope):
    # "stair": the staircase alone (survivals near 1: the break is the first
    # plateau edge inside the range); "stair_lin": the staircase times a linear
    # decay; "lin": a linear decay alone, which puts the break thousands of
    # candidates in (later tiles of the workspace path, which 1100 x 8 and
    # 3000 x 5 take).
    _say(f"case schedule early stop R={R} g={g} {kind} slope={slope}")
    from draft_head_step_amd.inputs import sps_table
    rng = np.random.default_rng(R + g)
    lo = 0.97 if kind == "stair" else 0.3
    a = O.survival(rng.uniform(lo, 1.0, size=(R, g)).astype(np.float32))
    B = np.arange(1, R * (1 + g) + 1, dtype=np.float64)
    lin = np.maximum(1.0 - slope * (B - 1), 0.01)
    stair = sps_table("staircase", R * (1 + g)).astype(np.float64)
    sps = (stair if kind == "stair" else lin if kind == "lin" else stair * lin).astype(np.float32)
    ref = _sched_ex_case(a, sps, D.SCHED_EARLY_STOP)
    assert 0 <= ref["m_star"] <= R * g


@pytest.mark.parametrize("R,g,K", [(4, 5, 0), (4, 5, 4), (4, 5, 13), (4, 5, 24), (4, 5, 99),
                                   (300, 5, 1000), (2000, 4, 9000), (2731, 3, 5000),
                                   (5000, 7, 20000), (5000, 7, 40000)])
def test_schedule_capacity(R, g, K):
    _say(f"case schedule capacity R={R} g={g} K={K}")
    rng = np.random.default_rng(K + R)
    a = O.survival(rng.uniform(0.05, 1.0, size=(R, g)).astype(np.float32))
    _sched_ex_case(a, None, D.SCHED_CAPACITY, K)


@pytest.mark.parametrize("R,g", [(700, 6), (3000, 6)])
def test_schedule_ex_ties_and_zeros(R, g):
    _say(f"case schedule ex ties R={R} g={g}")
    rng = np.random.default_rng(77)
    c = rng.choice(np.array([1.0, 0.5, 0.0, 0.75], np.float32), size=(R, g))
    a = O.survival(c)
    B = np.arange(1, R * (1 + g) + 1)
    sps = (0.999 ** (B / 64.0)).astype(np.float32)
    _sched_ex_case(a, sps, D.SCHED_EARLY_STOP)
    _sched_ex_case(a, None, D.SCHED_CAPACITY, R + (R * g) // 2)


# --------------------------------------------------------------------------- full sizes

def _sample_rows(R, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, R - 1], rng.choice(R, size=min(n, R), replace=False)]))


def _tile_rows(R, per_tile, seed):
    """`per_tile` random requests from every 32-request tile (so every wave's tile
    of every workgroup is checked), plus the first and last request."""
    rng = np.random.default_rng(seed)
    rows = [0, R - 1]
    for t0 in range(0, R, 32):
        n = min(32, R - t0)
        rows += list(t0 + rng.choice(n, size=min(per_tile, n), replace=False))
    return np.unique(np.asarray(rows))


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_qwen3_8b_full(layout):
    _say(f"case qwen3_8b (R=64, V=151936, r=256) layout={layout}")
    wl = make_workload(CONFIGS["qwen3_8b"])
    _full_path_check(wl, layout=layout)


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
def test_dsv4_full(layout, bias):
    # bias=False is the benchmarked call (no bias output).
    _say(f"case dsv4 (R=256, V=129280, r=512, sampling) layout={layout} bias={bias}")
    wl = make_workload(CONFIGS["dsv4"])
    _full_path_check(wl, rows=_tile_rows(256, 3, 1), layout=layout, bias_rows=bias)


def test_long_block_full():
    _say("case long_block (R=1024, gamma=16, V=129280, r=256)")
    wl = make_workload(CONFIGS["long_block"])
    g = H.to_device(wl, DEV)
    toks, _ = H.run_draft(wl, g, bias=False)
    H.check_draft(wl, toks, _tile_rows(1024, 1, 2))
    del g["base"]
    tok_dev = torch.from_numpy(toks).to(DEV)
    conf, surv = H.run_confidence(wl, g, tok_dev)
    H.check_confidence(wl, toks, conf, surv)
    lengths, order, info = H.run_schedule(torch.from_numpy(surv).to(DEV), g["sps"])
    H.check_schedule(surv, wl["sps"], lengths, order, info)


def test_step_events_time_each_fused_launch():
    _say("case step events")
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    ref, _ = H.run_draft(wl, g)
    gm = wl["base"].shape[1]
    begins = [torch.cuda.Event(enable_timing=True) for _ in range(gm)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(gm)]
    for e in begins + ends:
        e.record()   # materialise the hipEvent_t handles
    torch.cuda.synchronize()
    tok = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], wl["mode"],
                                wl["temperature"], None,
                                events=([e.cuda_event for e in begins], [e.cuda_event for e in ends]))
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), ref)
    for b, e in zip(begins, ends):
        ms = b.elapsed_time(e)
        assert 0.0 < ms < 100.0


# --------------------------------------------------------------------------- bias only

def _bias_only_case(wl, rows=None, bias=True, layout=D.LAYOUT_RGV):
    """base = NULL (greedy on the Markov bias alone) against the oracle with base = 0."""
    from draft_head_step_amd.inputs import from_tiled
    g = H.to_device(wl, DEV)
    R, gm, V = wl["base"].shape
    shape = (gm, (V + 31) // 32, 32, R) if layout == D.LAYOUT_TILED else (R, gm, V)
    bias_out = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV) if bias else None
    tok = D.dspark_markov_draft(g["W1"], g["W2"], None, g["anchors"], GREEDY, gamma=gm,
                                bias_out=bias_out, layout=layout)
    torch.cuda.synchronize()
    ref = dict(wl, base=np.zeros_like(wl["base"]), mode=GREEDY, uniforms=None)
    b = None
    if bias:
        b = bias_out.cpu().numpy()
        if layout == D.LAYOUT_TILED:
            b = from_tiled(b, V)
    H.check_draft(ref, tok.cpu().numpy(), rows, b)


@pytest.mark.parametrize("layout", [D.LAYOUT_RGV, D.LAYOUT_TILED])
@pytest.mark.parametrize("R,g,V,r", [(4, 5, 4096, 64), (70, 4, 3000, 256), (3, 6, 64, 512),
                                     (300, 2, 777, 64)])
def test_bias_only_small(R, g, V, r, layout):
    _say(f"case bias-only R={R} g={g} V={V} r={r} layout={layout}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=r, d=16, mode=GREEDY, temperature=1.0, w_std=0.3,
                 base_std=1.0, wconf_std=0.1, seed=500 + R)
    _bias_only_case(make_workload(cfg), layout=layout)


@pytest.mark.parametrize("R,g,V,r", [(130, 3, 3000, 256), (600, 2, 5000, 128),
                                     (1024, 2, 20000, 256)])
def test_bias_only_two_tiles_per_wave(R, g, V, r):
    # No bias output, ranks 128-256, >= 128 requests: each wave carries two
    # 32-request tiles (one partial R block, two blocks with a partial second,
    # full blocks).
    _say(f"case bias-only two tiles R={R} g={g} V={V} r={r}")
    cfg = Config("edge", R=R, gamma=g, V=V, r=r, d=16, mode=GREEDY, temperature=1.0, w_std=0.3,
                 base_std=1.0, wconf_std=0.1, seed=700 + R)
    _bias_only_case(make_workload(cfg), bias=False)


def test_bias_only_long_block_shape():
    # R = 1024, r = 256, V = 129280 (two of the 16 positions), sampled rows.
    _say("case bias-only at R=1024, V=129280, r=256")
    from draft_head_step_amd.inputs import make_head
    hd = make_head(CONFIGS["long_block"])
    R, V, gm = hd["R"], hd["V"], 2
    wl = {"W1": hd["W1"], "W2": hd["W2"], "anchors": hd["anchors"], "mode": GREEDY,
          "temperature": 1.0, "uniforms": None,
          "base": np.zeros((R, gm, V), np.float32)}   # pages touched only for sampled rows
    g = H.to_device({k: wl[k] for k in ("W1", "W2", "anchors")}, DEV)
    tok = D.dspark_markov_draft(g["W1"], g["W2"], None, g["anchors"], GREEDY, gamma=gm)
    torch.cuda.synchronize()
    H.check_draft(wl, tok.cpu().numpy(), rows=_sample_rows(R, 16, 6))


def test_bias_only_dsv4_shape():
    _say("case bias-only at R=256, V=129280, r=512")
    cfg = dataclasses.replace(CONFIGS["dsv4"], mode=GREEDY, w_std=0.05)
    _bias_only_case(make_workload(cfg), rows=_sample_rows(256, 16, 4), bias=False)


def test_stream_argument_that_is_not_current():
    # Calls given a stream that is not the current one: the binding's own
    # allocations (outputs, workspaces) are made on that stream, and the results
    # equal those of calls on the current stream.
    _say("case non-current stream argument")
    wl = make_workload(CONFIGS["tiny"], w_std=0.3)
    g = H.to_device(wl, DEV)
    ref_t = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], GREEDY)
    ref_c, ref_s = D.dspark_confidence(g["h"], g["W1"], g["anchors"], ref_t, g["w_conf"])
    ref_l, ref_o, _ = D.dspark_schedule(ref_s, g["sps"], want_order=True)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    assert torch.cuda.current_stream() != st
    for _ in range(3):
        t = D.dspark_markov_draft(g["W1"], g["W2"], g["base"], g["anchors"], GREEDY, stream=st)
        c, s = D.dspark_confidence(g["h"], g["W1"], g["anchors"], t, g["w_conf"], stream=st)
        l, o, info = D.dspark_schedule(s, g["sps"], want_order=True, want_info=True, stream=st)
        st.synchronize()
        assert torch.equal(t, ref_t) and torch.equal(c, ref_c) and torch.equal(s, ref_s)
        assert torch.equal(l, ref_l) and torch.equal(o, ref_o)
        assert D.schedule_info(info).m_star == O.schedule(ref_s.cpu().numpy(), wl["sps"])["m_star"]
