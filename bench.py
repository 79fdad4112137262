"""Benchmark: draft tokens/s of the DSpark drafter hot path on one MI355X.

One step = one dspark_draft_step call over one batch that is already resident
in HBM: the gamma fused refinement steps of the Markov-head draft, the
confidence head with STS and survival, and the global-search schedule
(tau * SPS(B) over every budget).  The default workload is the
DeepSeek-V4-shaped drafter: R = 256 requests, gamma = 5, V = 129280, Markov
rank r = 512, hidden d = 7168, Gumbel-max sampling at T = 1.

The base logits and uniforms are handed over row-major ([R][gamma][V]) by
default; the column-tiled layout ([gamma][ceil(V/32)][32][R]), the three
separate entry points, and the same call re-using one weight copy (so that
W2 stays in the Infinity Cache from call to call) are timed in the same run
and reported beside it.  The headline steps take several copies of W1/W2 in
turn, so no step finds W2 left in the Infinity Cache by the step before, as
in a serving loop where the target model runs between two drafting calls.

Prints one JSON line with the throughput, the roofline position of the
dominant kernel (the fused Markov step, timed live with HIP events on the
stream it runs on), and the CPU oracle's throughput on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
METRIC = "draft tokens/s (Markov refine+confidence+schedule) at R=256,V=129280; % roofline"
COUNTERS_FMT = os.path.join(ROOT, "profiles", "markov_step_{cfg}_{layout}_counters.txt")


STEP_SOURCES = ["markov_kernels.h", "markov_types.h", "packed_words.h", "markov_step.hip",
                "markov_pick_greedy_row.hip", "markov_pick_greedy_col.hip",
                "markov_pick_sample_row.hip", "markov_pick_sample_col.hip",
                "markov_pick_bias_only.hip", "dspark_internal.h", "sched_lds.h"]


def source_hash():
    """Hash of the sources and flags of the fused step kernels (what the counters
    measure): a change to any other part of the library leaves them valid."""
    import hashlib
    from draft_head_step_amd import build
    h = hashlib.sha256()
    for name in STEP_SOURCES:
        with open(os.path.join(build.CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(build.HIPCC_FLAGS).encode())
    return h.hexdigest()[:32]


def step_bytes(wl) -> int:
    """Algorithmic HBM bytes of one fused Markov step (one launch, all R requests):
    W2 once, the base logits of this position, the uniforms (sampling), the
    gathered W1 rows and the previous-token ids."""
    R, g, V = wl["base"].shape
    r = wl["W1"].shape[1]
    b = V * r * 2 + R * V * 4 + R * r * 2 + R * 4
    if wl["uniforms"] is not None:
        b += R * V * 4
    return b


def whole_step_bytes(wl) -> int:
    """Algorithmic HBM bytes of one whole step: gamma fused Markov steps, the
    confidence head (h, the gathered W1 rows, w, conf and surv written), and the
    schedule (survivals read, the SPS entries B = R .. R(1+gamma), lengths)."""
    R, g, V = wl["base"].shape
    r = wl["W1"].shape[1]
    d = wl["h"].shape[2]
    conf = R * g * d * 2 + R * g * r * 2 + (d + r) * 4 + 2 * R * g * 4
    sched = R * g * 4 + (R * g + 1) * 4 + R * 4
    return g * step_bytes(wl) + conf + sched


def read_traffic(cfg, layout):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if the counters were taken on a different version of the library source."""
    path = COUNTERS_FMT.format(cfg=cfg, layout=layout)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("step_source_hash") != source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def device_workload(cfg, dev, seed=None):
    """Inputs of ``cfg`` drawn on the device (seeded torch generator) with the same
    shapes and distributions as draft_head_step_amd.inputs.make_workload; used
    for timing-only configurations whose logits are too large to draw on the
    host quickly (the parity tests use the host workloads)."""
    import torch
    from draft_head_step_amd.inputs import sps_table
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed if seed is None else seed)
    R, g, V, r, d = cfg.R, cfg.gamma, cfg.V, cfg.r, cfg.d

    def normal(shape, std):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).mul_(std)

    base = normal((R, g, V), cfg.base_std)
    if cfg.boost_count:
        ids = torch.randint(0, V, (R, g, cfg.boost_count), generator=gen, device=dev)
        base.scatter_(2, ids, base.gather(2, ids) + cfg.boost_value)
    uniforms = None
    if cfg.mode == 1:
        k = torch.randint(0, 1 << 23, (R, g, V), generator=gen, device=dev, dtype=torch.int32)
        uniforms = k.to(torch.float32).add_(0.5).mul_(2.0 ** -23)
    b_max = max(cfg.b_max, R * (1 + g))
    return {"R": R, "gamma": g, "V": V, "r": r, "d": d, "mode": cfg.mode,
            "temperature": cfg.temperature,
            "W1": normal((V, r), cfg.w_std).to(torch.bfloat16),
            "W2": normal((V, r), cfg.w_std).to(torch.bfloat16),
            "base": base, "uniforms": uniforms,
            "h": normal((R, g, d), cfg.h_std).to(torch.bfloat16),
            "w_conf": normal((d + r,), cfg.wconf_std),
            "anchors": torch.randint(0, V, (R,), generator=gen, device=dev, dtype=torch.int32),
            "sts": None if cfg.sts is None else torch.tensor(cfg.sts, dtype=torch.float32,
                                                               device=dev),
            "sps": torch.from_numpy(sps_table(cfg.sps_kind, b_max)).to(dev)}


def tiled_on_device(x):
    """[R, gamma, V] -> column-tiled [gamma, ceil(V/32), 32, R] on the device (tail entries zero)."""
    import torch
    R, g, V = x.shape
    C = (V + 31) // 32
    if C * 32 != V:
        x = torch.nn.functional.pad(x, (0, C * 32 - V))
    return x.view(R, g, C, 32).permute(1, 2, 3, 0).contiguous()


def cpu_baseline(wl, min_s=10.0, max_calls=20):
    """Time the CPU oracle (as it stands) on whole calls of the same workload, repeated
    until about min_s seconds of CPU work have passed (at most max_calls calls)."""
    from oracle import dspark_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    R, g, _ = wl["base"].shape
    calls = 0
    t0 = time.perf_counter()
    while calls < max_calls:
        O.run_path(wl)
        calls += 1
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    return {"value": calls * R * g / dt, "unit": "draft tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{calls} full calls (each all {R} requests x {g} positions: draft, "
                      f"confidence, survival, schedule) in {dt:.1f} s, numpy fp64 oracle, "
                      f"BLAS threads={threads}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prewarm-ms", type=float, default=60.0,
                    help="time-based warm-up before the counted warm-up steps (the GPU "
                         "reaches its sustained clocks only after ~20 ms of work)")
    ap.add_argument("--config", default="dsv4")
    ap.add_argument("--layout", choices=["tiled", "rgv"], default="rgv",
                    help="storage order of base / uniforms handed to the draft")
    ap.add_argument("--path", choices=["fused", "calls"], default="fused",
                    help="one dspark_draft_step call per step, or the three separate calls")
    ap.add_argument("--weight-copies", type=int, default=-1,
                    help="copies of W1/W2 the steps take in turn (default: enough that three "
                         "times the 256 MB Infinity Cache separates two uses of one copy)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the side measurements (same weights, other layout, three calls, "
                         "cold caches, GEMM-only, scheduler stress, other configurations, "
                         "measured bandwidth)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["gemm", "rnn", "sched", "verify", "conf"],
                    help="run one side measurement alone and print its JSON (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no "
              "multi-GPU mode (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_head_step_amd as D
    from draft_head_step_amd.inputs import CONFIGS, make_head, make_workload, to_tiled

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # A plain copy of known size: reads and writes exactly 1 GiB per dispatch.
        n = (1 << 30) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": n * 4, "dispatches": 3}), flush=True)
        return
    stream = torch.cuda.current_stream()

    def warm(fn, ms=40.0):
        """Run fn until about `ms` of GPU work has passed (sustained clocks)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()

    def scheduler_only(calls=30):
        """dspark_survival + the schedule on the scheduler stress workload (R = 8192,
        gamma = 7, SPS over B = 1..65536): microseconds per call from HIP events, for
        the global search (dspark_schedule) and for dspark_schedule_ex's early-stop
        and capacity rules (capacity: half of the candidates)."""
        sw = make_workload(CONFIGS["sched_stress"])
        sc = torch.from_numpy(sw["conf"]).to(dev)
        ssps = torch.from_numpy(sw["sps"]).to(dev)
        sR, sg = sw["conf"].shape
        ssurv = torch.empty_like(sc)
        slen = torch.empty((sR,), dtype=torch.int32, device=dev)
        sws = torch.empty(D.dspark_schedule_workspace(sR, sg), dtype=torch.uint8, device=dev)
        cap = sR + sR * sg // 2

        def timed(sched):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(calls)]

            def one():
                D.dspark_survival(sc, surv=ssurv, stream=stream)
                sched()
            warm(one, 20.0)
            us = []
            for b, e in evs:
                b.record(stream)
                one()
                e.record(stream)
                torch.cuda.synchronize()
                us.append(b.elapsed_time(e) * 1e3)
            return [round(float(x), 1) for x in np.percentile(us, [10, 50, 90])]

        glob = timed(lambda: D.dspark_schedule(ssurv, ssps, lengths=slen, workspace=sws,
                                               stream=stream))
        early = timed(lambda: D.dspark_schedule_ex(ssurv, ssps, mode=D.SCHED_EARLY_STOP,
                                                   lengths=slen, workspace=sws, stream=stream))
        capy = timed(lambda: D.dspark_schedule_ex(ssurv, None, mode=D.SCHED_CAPACITY,
                                                  capacity=cap, lengths=slen, workspace=sws,
                                                  stream=stream))
        nbytes = sR * sg * 4 * 2 + sw["sps"].nbytes + sR * 4
        return {"workload": f"sched_stress: R={sR}, gamma={sg}, B_max={sw['B_max']}",
                "us_per_call_p10_p50_p90": glob,
                "early_stop_us_p10_p50_p90": early,
                "capacity_us_p10_p50_p90": capy, "capacity_K": cap,
                "algorithmic_bytes": int(nbytes),
                "achieved_GBps_at_p50": round(nbytes / (glob[1] / 1e6) / 1e9, 2),
                "bound": "latency (launches: 1 survival + 11 schedule)"}

    cfg = CONFIGS[args.config]
    if cfg.beta_means is not None:
        # Scheduler-only workload: survival + schedule per call.
        res = scheduler_only(calls=args.steps)
        p50 = res["us_per_call_p10_p50_p90"][1]
        print(json.dumps({"metric": "schedule latency (survival + schedule) per call",
                          "value": p50, "unit": "us", "n_gpus": 1, "steps": args.steps,
                          "warmup": "20 ms", "higher_is_better": False, "dtype": "f32/u64",
                          "data": "synthetic", "config": {"workload": res["workload"]},
                          "scheduler": res}), flush=True)
        return
    wl = make_workload(cfg)
    R, g, V = wl["base"].shape
    r = wl["W1"].shape[1]
    d = wl["h"].shape[2]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    W1, W2, h = bf16(wl["W1"]), bf16(wl["W2"]), bf16(wl["h"])
    layouts = {"tiled": D.LAYOUT_TILED, "rgv": D.LAYOUT_RGV}

    def inputs(layout):
        conv = to_tiled if layout == "tiled" else (lambda a: a)
        b = torch.from_numpy(conv(wl["base"])).to(dev)
        u = torch.from_numpy(conv(wl["uniforms"])).to(dev) if wl["uniforms"] is not None else None
        return b, u
    anchors = torch.from_numpy(wl["anchors"]).to(dev)
    w_conf = torch.from_numpy(wl["w_conf"]).to(dev)
    sts = torch.from_numpy(wl["sts"]).to(dev) if wl["sts"] is not None else None
    sps = torch.from_numpy(wl["sps"]).to(dev)
    tokens = torch.empty((R, g), dtype=torch.int32, device=dev)
    conf = torch.empty((R, g), dtype=torch.float32, device=dev)
    surv = torch.empty((R, g), dtype=torch.float32, device=dev)
    lengths = torch.empty((R,), dtype=torch.int32, device=dev)
    ws_d = torch.empty(D.dspark_markov_draft_workspace(R, g, V, r), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(D.dspark_schedule_workspace(R, g), dtype=torch.uint8, device=dev)

    prewarm_ms = max(float(args.prewarm_ms), 0.0)

    def weight_copies(W1_, W2_, n):
        """n copies of the head's weights in separate device memory (copy 0 is the
        original).  Steps take them in turn, so no call finds its W2 left in the
        256 MB Infinity Cache by the call before it, as in a serving loop where
        the target model's forward pass runs between two drafting calls."""
        out = [(W1_, W2_)]
        for _ in range(n - 1):
            out.append((W1_.clone(), W2_.clone()))
        return out

    def copies_for(w2_bytes):
        return max(4, -(-3 * (256 << 20) // w2_bytes))

    n_copies = copies_for(V * r * 2) if args.weight_copies < 0 else max(args.weight_copies, 1)
    heads = weight_copies(W1, W2, n_copies)
    ws_f = torch.empty(D.dspark_draft_step_workspace(R, g, V, r), dtype=torch.uint8, device=dev)

    def make_step(path, layout, base, unif):
        lay = layouts[layout]

        def one_step(i, ev=None):
            hW1, hW2 = heads[i % len(heads)]
            if path == "fused":
                D.dspark_draft_step(hW1, hW2, base, anchors, h, w_conf, sps, wl["mode"],
                                    wl["temperature"], unif, sts_temp=sts, tokens=tokens, conf=conf,
                                    surv=surv, lengths=lengths, workspace=ws_f, events=ev,
                                    stream=stream, layout=lay)
            else:
                D.dspark_markov_draft(hW1, hW2, base, anchors, wl["mode"], wl["temperature"],
                                      unif, tokens=tokens, workspace=ws_d, events=ev,
                                      stream=stream, layout=lay)
                D.dspark_confidence(h, hW1, anchors, tokens, w_conf, sts, conf=conf, surv=surv,
                                    stream=stream)
                D.dspark_schedule(surv, sps, lengths=lengths, workspace=ws_s, stream=stream)
        return one_step

    def run(path, layout, steps, warmup, ev_steps=50, copies=None):
        """Time `steps` whole steps; return (ms per step, fused-step launch durations in
        ms as [ev_steps][gamma]).

        Everything the timed region needs (events included) is made before the
        warm-up, and the timed steps follow the warm-up at once: the GPU runs at
        its sustained clocks (after an idle gap the first ~20 ms of steps run
        about 10% slower; the time-based pre-warm covers that whatever the
        counted warm-up).  The per-launch durations come from a second run of
        `ev_steps` steps with HIP events attached to each fused launch's dispatch."""
        nonlocal heads
        saved = heads
        if copies is not None:
            heads = heads[:copies]
        base, unif = inputs(layout)
        one_step = make_step(path, layout, base, unif)

        def mk():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)   # materialise the underlying hipEvent_t
            return e
        begins = [[mk() for _ in range(g)] for _ in range(ev_steps)]
        ends = [[mk() for _ in range(g)] for _ in range(ev_steps)]
        evs = [([e.cuda_event for e in begins[i]], [e.cuda_event for e in ends[i]])
               for i in range(ev_steps)]
        torch.cuda.synchronize()

        cnt = [0]

        def next_step():
            one_step(cnt[0])
            cnt[0] += 1
        warm(next_step, prewarm_ms)
        for _ in range(warmup):
            next_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            next_step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # HIP events bracketing every fused Markov step launch.
        for i in range(ev_steps):
            one_step(cnt[0], evs[i])
            cnt[0] += 1
        torch.cuda.synchronize()
        durs = np.array([[begins[i][k].elapsed_time(ends[i][k]) for k in range(g)]
                         for i in range(ev_steps)])
        del base, unif
        heads = saved
        return (t1 - t0) * 1e3 / steps, durs

    def graph_steps(layout, steps, warmup):
        """ms per step with the fused call captured in a HIP graph (one graph per
        weight copy, taken in turn as in the timed steps) and replayed."""
        base, unif = inputs(layout)
        lay = layouts[layout]

        def call(i):   # on the current stream: the capture stream inside torch.cuda.graph
            hW1, hW2 = heads[i % len(heads)]
            D.dspark_draft_step(hW1, hW2, base, anchors, h, w_conf, sps, wl["mode"],
                                wl["temperature"], unif, sts_temp=sts, tokens=tokens, conf=conf,
                                surv=surv, lengths=lengths, workspace=ws_f, layout=lay)
        for i in range(len(heads)):
            call(i)
        torch.cuda.synchronize()
        graphs = []
        for i in range(len(heads)):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                call(i)
            graphs.append(gr)
        torch.cuda.synchronize()
        cnt = [0]

        def next_replay():
            graphs[cnt[0] % len(graphs)].replay()
            cnt[0] += 1
        warm(next_replay, prewarm_ms)
        for _ in range(warmup):
            next_replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            next_replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del graphs, base, unif
        return (t1 - t0) * 1e3 / steps

    def cold_steps(layout, n):
        """Per-step time of the fused call with the caches flushed first (a 512 MB
        read, outside the bracketed step, so no dirty lines are written back
        inside it): median over n steps, in ms, and the median duration of the
        fused launch at each position (position 1 reads W2 cold; later positions
        may find it in the 256 MB Infinity Cache)."""
        base, unif = inputs(layout)
        one_step = make_step("fused", layout, base, unif)
        scratch = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)

        def mk():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        evs = [(mk(), mk()) for _ in range(n + 1)]
        kb = [[mk() for _ in range(g)] for _ in range(n + 1)]
        ke = [[mk() for _ in range(g)] for _ in range(n + 1)]
        warm(lambda: torch.sum(scratch, dim=0, out=sink))
        times, per_pos = [], []
        for i in range(n + 1):
            torch.sum(scratch, dim=0, out=sink)
            b, e = evs[i]
            b.record(stream)
            one_step(0, ([x.cuda_event for x in kb[i]], [x.cuda_event for x in ke[i]]))
            e.record(stream)
            torch.cuda.synchronize()
            if i:
                times.append(b.elapsed_time(e))
                per_pos.append([kb[i][k].elapsed_time(ke[i][k]) for k in range(g)])
        del base, unif, scratch
        pos_us = [round(float(x) * 1e3, 2) for x in np.median(np.asarray(per_pos), axis=0)]
        return float(np.median(times)), pos_us

    def gemm_only(name, steps=10):
        """Greedy on the Markov bias alone (no logits stream): the gather + bias GEMM +
        argmax, per fused launch, against the bf16 MFMA peak."""
        c = CONFIGS[name]
        hd = make_head(c)
        gW1, gW2 = bf16(hd["W1"]), bf16(hd["W2"])
        ganc = torch.from_numpy(hd["anchors"]).to(dev)
        gR, gg, gV, gr = hd["R"], hd["gamma"], hd["V"], hd["r"]
        gtok = torch.empty((gR, gg), dtype=torch.int32, device=dev)
        gws = torch.empty(D.dspark_markov_draft_workspace(gR, gg, gV, gr), dtype=torch.uint8,
                          device=dev)
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(gg)] for _ in range(steps)]
        eve = [[torch.cuda.Event(enable_timing=True) for _ in range(gg)] for _ in range(steps)]
        for lst in evb + eve:
            for e in lst:
                e.record(stream)
        warm(lambda: D.dspark_markov_draft(gW1, gW2, None, ganc, 0, gamma=gg, tokens=gtok,
                                           workspace=gws, stream=stream))
        for i in range(steps):
            D.dspark_markov_draft(gW1, gW2, None, ganc, 0, gamma=gg, tokens=gtok, workspace=gws,
                                  stream=stream,
                                  events=([e.cuda_event for e in evb[i]], [e.cuda_event for e in eve[i]]))
        torch.cuda.synchronize()
        ms = float(np.mean([evb[i][k].elapsed_time(eve[i][k])
                            for i in range(steps) for k in range(gg)]))
        flops = 2.0 * gR * gr * gV
        tf = flops / (ms / 1e3) / 1e12
        del gW1, gW2, gws
        return {"shape": f"{name}: R={gR}, r={gr}, V={gV}", "avg_launch_ms": round(ms, 5),
                "tflops": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}

    def whole_step_config(name, steps=20):
        """Another configuration's whole step (the fused call) with inputs drawn on
        the device, in the headline layout, weight copies taken in turn; per-step
        ms and fused-launch us."""
        c = CONFIGS[name]
        w = device_workload(c, dev)
        cR, cg, cV, cr = w["R"], w["gamma"], w["V"], w["r"]
        cb = tiled_on_device(w["base"]) if args.layout == "tiled" else w["base"]
        cu = w["uniforms"]
        if cu is not None and args.layout == "tiled":
            cu = tiled_on_device(cu)
        w["base"] = w["uniforms"] = None
        lay = layouts[args.layout]
        ch = weight_copies(w["W1"], w["W2"], copies_for(cV * cr * 2))
        ctok = torch.empty((cR, cg), dtype=torch.int32, device=dev)
        cconf = torch.empty((cR, cg), dtype=torch.float32, device=dev)
        csurv = torch.empty((cR, cg), dtype=torch.float32, device=dev)
        clen = torch.empty((cR,), dtype=torch.int32, device=dev)
        cws = torch.empty(D.dspark_draft_step_workspace(cR, cg, cV, cr), dtype=torch.uint8,
                          device=dev)
        cnt = [0]

        def one(ev=None):
            hW1, hW2 = ch[cnt[0] % len(ch)]
            cnt[0] += 1
            D.dspark_draft_step(hW1, hW2, cb, w["anchors"], w["h"], w["w_conf"], w["sps"], c.mode,
                                c.temperature, cu, sts_temp=w["sts"], tokens=ctok, conf=cconf,
                                surv=csurv, lengths=clen, workspace=cws, events=ev, stream=stream,
                                layout=lay)

        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(cg)] for _ in range(steps)]
        eve = [[torch.cuda.Event(enable_timing=True) for _ in range(cg)] for _ in range(steps)]
        for lst in evb + eve:
            for e in lst:
                e.record(stream)
        warm(one)
        t0 = time.perf_counter()
        for _ in range(steps):
            one()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        for i in range(steps):
            one(([e.cuda_event for e in evb[i]], [e.cuda_event for e in eve[i]]))
        torch.cuda.synchronize()
        kd = [evb[i][k].elapsed_time(eve[i][k]) for i in range(steps) for k in range(cg)]
        kms = float(np.mean(kd))
        nb = cV * cr * 2 + cR * cV * 4 * (2 if cu is not None else 1) + cR * cr * 2 + cR * 4
        nch = len(ch)
        del w, cb, cu, cws, ch
        return {"workload": f"{name}: R={cR}, gamma={cg}, V={cV}, r={cr}, d={c.d}, "
                            f"{'sampling' if c.mode else 'greedy'}, layout {args.layout}",
                "ms_per_step": round(ms, 4), "value": round(cR * cg / (ms / 1e3), 1),
                "unit": "draft tokens/s", "avg_launch_ms": round(kms, 5),
                "launch_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(kd, [10, 50, 90])],
                "frac": round(nb / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "weight_copies": nch,
                "data": "synthetic, drawn on the device (seeded torch generator)"}

    def verify_side(vR=256, vg=5, vV=129280, calls=20):
        """The verification side at the DeepSeek-V4 shape, every request keeping all
        gamma drafts (B = R (1 + gamma) flattened elements): dspark_verify_pack,
        dspark_verify_greedy over the B target rows, and dspark_accept_prob over
        R * gamma draft / target row pairs.  Inputs drawn on the device."""
        gen = torch.Generator(device=dev)
        gen.manual_seed(21)
        anc = torch.randint(0, vV, (vR,), generator=gen, device=dev, dtype=torch.int32)
        drafts = torch.randint(0, vV, (vR, vg), generator=gen, device=dev, dtype=torch.int32)
        lens = torch.full((vR,), vg, dtype=torch.int32, device=dev)
        nB = vR * (1 + vg)
        tgt = torch.randn((nB, vV), generator=gen, device=dev).mul_(2.0)
        dl = torch.randn((vR * vg, vV), generator=gen, device=dev).mul_(3.0)
        tl = dl + torch.randn((vR * vg, vV), generator=gen, device=dev)
        ft = torch.empty((nB,), dtype=torch.int32, device=dev)
        fpos = torch.empty_like(ft)
        freq = torch.empty_like(ft)
        cu = torch.empty((vR + 1,), dtype=torch.int32, device=dev)
        am = torch.empty((nB,), dtype=torch.int32, device=dev)
        acc = torch.empty((vR,), dtype=torch.int32, device=dev)
        nxt = torch.empty((vR,), dtype=torch.int32, device=dev)
        ap = torch.empty((vR * vg,), dtype=torch.float32, device=dev)

        def timed(fn):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(calls)]
            warm(fn, 20.0)
            for b, e in evs:
                b.record(stream)
                fn()
                e.record(stream)
            torch.cuda.synchronize()
            return float(np.median([b.elapsed_time(e) for b, e in evs])) * 1e3

        pack = lambda: D.dspark_verify_pack(anc, drafts, lens, flat_tokens=ft, flat_pos=fpos,
                                            flat_req=freq, cu_seqlens=cu, stream=stream)
        pack()
        us_pack = timed(pack)
        us_greedy = timed(lambda: D.dspark_verify_greedy(tgt, cu, drafts, target_argmax=am,
                                                         accepted=acc, next_token=nxt,
                                                         stream=stream))
        us_acc = timed(lambda: D.dspark_accept_prob(dl, tl, 1.0, out=ap, stream=stream))
        b_greedy = nB * vV * 4
        b_acc = 2 * vR * vg * vV * 4
        del tgt, dl, tl
        return {"workload": f"R={vR}, gamma={vg}, V={vV}, every draft kept (B={nB})",
                "pack_us": round(us_pack, 1),
                "greedy_us": round(us_greedy, 1),
                "greedy_frac_of_hbm": round(b_greedy / (us_greedy / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                "accept_prob_us": round(us_acc, 1),
                "accept_prob_frac_of_hbm": round(b_acc / (us_acc / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "fractions use one read of the logits (the accept-prob kernel keeps "
                        "about half of each row pair on chip between its max/sum and min-sum "
                        "passes and reads the rest twice)"}

    def confidence_side(calls=50):
        """dspark_confidence (with survival) on the default workload's tokens, timed
        alone with HIP events around each call: us per call and the fraction of the
        HBM peak on its algorithmic bytes (h, the gathered W1 rows, w, the outputs)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        fn = lambda: D.dspark_confidence(h, W1, anchors, tokens, w_conf, sts, conf=conf, surv=surv,
                                         stream=stream)
        warm(fn, 20.0)
        for b, e in evs:
            b.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        us = [b.elapsed_time(e) * 1e3 for b, e in evs]
        p50 = float(np.median(us))
        # The same calls back to back without the host in between: captured in one
        # HIP graph (each call only enqueues its kernel) and replayed between one
        # event pair, so each launch is queued while the previous call runs.
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(graph, stream=gs):
                for _ in range(calls):
                    D.dspark_confidence(h, W1, anchors, tokens, w_conf, sts, conf=conf, surv=surv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        b2b = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        b2b[0].record()
        graph.replay()
        b2b[1].record()
        torch.cuda.synchronize()
        us_b2b = b2b[0].elapsed_time(b2b[1]) * 1e3 / calls
        del graph
        nb = R * g * d * 2 + R * g * r * 2 + (d + r) * 4 + 2 * R * g * 4
        return {"workload": f"{cfg.name}: R={R}, gamma={g}, d={d}, r={r}",
                "us_per_call_p10_p50_p90": [round(float(x), 2) for x in np.percentile(us, [10, 50, 90])],
                "us_per_call_back_to_back": round(us_b2b, 2),
                "algorithmic_bytes": int(nb),
                "achieved_GBps_back_to_back": round(nb / (us_b2b / 1e6) / 1e9, 1),
                "frac_of_hbm": round(nb / (us_b2b / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_of_hbm_single_call_p50": round(nb / (p50 / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "frac_of_hbm: calls back to back from a HIP graph (launch queued "
                        "behind the previous call, no host in between); the percentiles time "
                        "one call per event pair from the host, launch included. Every call "
                        "reads the same h (18.4 MB), which the Infinity Cache can hold, as it "
                        "would hold hidden states the backbone has just written"}

    def rnn_side(calls=20):
        """dspark_rnn_draft on the default workload (the RNN head's alternative
        sequential stage, same W1 / W2 / logits, seeded head weights U, b): per
        call ms and the step kernels' launch durations from HIP events; the
        pre-activation and state-update kernels take the rest of the call."""
        from draft_head_step_amd.inputs import make_rnn_head
        hd = make_rnn_head(cfg)
        U = bf16(hd["U"])
        b = torch.from_numpy(hd["b"]).to(dev)
        base, unif = inputs(args.layout)
        lay = layouts[args.layout]
        rws = torch.empty(D.dspark_rnn_draft_workspace(R, g, V, r, d), dtype=torch.uint8, device=dev)
        cnt = [0]

        def one(ev=None):
            hW1, hW2 = heads[cnt[0] % len(heads)]
            cnt[0] += 1
            D.dspark_rnn_draft(hW1, hW2, U, b, base, h, anchors, wl["mode"], wl["temperature"],
                               unif, tokens=tokens, workspace=rws, events=ev, stream=stream,
                               layout=lay)
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(g)] for _ in range(calls)]
        eve = [[torch.cuda.Event(enable_timing=True) for _ in range(g)] for _ in range(calls)]
        cb = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
        for lst in evb + eve + [cb, ce]:
            for e in lst:
                e.record(stream)
        warm(one, 20.0)
        for i in range(calls):
            cb[i].record(stream)
            one(([e.cuda_event for e in evb[i]], [e.cuda_event for e in eve[i]]))
            ce[i].record(stream)
        torch.cuda.synchronize()
        call_ms = float(np.median([cb[i].elapsed_time(ce[i]) for i in range(calls)]))
        step_ms = float(np.mean([evb[i][k].elapsed_time(eve[i][k])
                                 for i in range(calls) for k in range(g)]))
        flops_pre = 2.0 * R * g * d * 2 * r
        flops_state = 2.0 * R * 2 * r * 2 * r * g
        del base, unif, rws, U
        return {"workload": f"{cfg.name} shapes, RNN head (U [2r, 2r + d] bf16), layout {args.layout}",
                "ms_per_call_median": round(call_ms, 4),
                "value": round(R * g / (call_ms / 1e3), 1), "unit": "draft tokens/s",
                "step_kernel_avg_ms": round(step_ms, 5),
                "step_kernel_frac_of_hbm": round(nbytes / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "launches_per_call": 2 * g + 2,
                "recurrent_gemm_flops_per_call": flops_pre + flops_state,
                "note": "events on the step kernels only; the call also runs the pre-activation "
                        "GEMM and gamma state updates (rocprofv3 summary in profiles/)"}

    def hbm_measured(nbytes=1 << 31, reps=5):
        """Large-copy bandwidth (read + write bytes over time) of torch's device copy:
        a measured reference beside the published peak."""
        n = nbytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        ts = []
        for _ in range(reps):
            b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b.record(stream)
            dst.copy_(src)
            e.record(stream)
            torch.cuda.synchronize()
            ts.append(b.elapsed_time(e))
        del src, dst
        return {"copy_GBps": round(2 * nbytes / (float(np.median(ts)) / 1e3) / 1e9, 1),
                "bytes_copied": nbytes}

    nbytes = step_bytes(wl)
    if args.only:
        def conf_only():
            # seeded valid ids in place of a draft's tokens
            gen = torch.Generator(device="cpu").manual_seed(7)
            tokens.copy_(torch.randint(0, wl["W1"].shape[0], (R, g), generator=gen,
                                       dtype=torch.int32))
            return confidence_side(calls=max(args.steps, 50))
        res = {"gemm": lambda: [gemm_only(args.config), gemm_only("long_block")],
               "rnn": rnn_side, "sched": scheduler_only, "verify": verify_side,
               "conf": conf_only}[args.only]()
        print(json.dumps({"only": args.only, "result": res}), flush=True)
        return
    ms_per_step, durs = run(args.path, args.layout, args.steps, args.warmup)
    k_ms = float(np.mean(durs))
    pos_ms = durs.mean(axis=0)
    value = R * g / (ms_per_step / 1e3)
    achieved = nbytes / (k_ms / 1e3) / 1e9
    # The library runs rank-512 sampling on the K-split kernel, everything else
    # on the plain one; the fused call's last step may be the K-split kernel
    # that also does the finishing work (the launch count says which).
    kernel = "markov_step_ksplit_kernel" if (r > 256 and wl["mode"]) else "markov_step_kernel"
    whole = whole_step_bytes(wl)
    if args.path == "fused":
        launches = D.dspark_draft_step_launches(R, g, V, r, layouts[args.layout], wl["mode"],
                                                wl["temperature"])
        if kernel == "markov_step_ksplit_kernel" and launches == g + 1:
            kernel = "markov_step_ksplit_kernel (last step: markov_step_ksplit_fin_kernel)"
    else:
        launches = g + 4

    def summary(ms, dd):
        km = float(np.mean(dd))
        return {"ms_per_step": round(ms, 4), "value": round(R * g / (ms / 1e3), 1),
                "avg_launch_ms": round(km, 5),
                "frac": round(nbytes / (km / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "whole_step_frac_of_hbm": round(whole / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: R={R}, gamma={g}, V={V}, r={r}, d={d}, "
                               f"{'Gumbel-max sampling T=%g' % wl['temperature'] if wl['mode'] else 'greedy'}",
                   "R": R, "gamma": g, "V": V, "r": r, "d": d, "layout": args.layout,
                   "call": "dspark_draft_step" if args.path == "fused"
                           else "dspark_markov_draft + dspark_confidence + dspark_schedule",
                   "launches_per_step": launches, "weight_copies": n_copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(cfg.name, args.layout),
                     "kernel": kernel, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_ms": round(k_ms, 5), "launches_per_step": g,
                     "launch_ms_p10_p50_p90": [round(float(x), 5)
                                               for x in np.percentile(durs, [10, 50, 90])],
                     "avg_launch_ms_by_position": [round(float(x), 5) for x in pos_ms],
                     "mfma_frac": round(2.0 * R * r * V / (k_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "whole_step": {"algorithmic_bytes": whole,
                       "achieved_GBps": round(whole / (ms_per_step / 1e3) / 1e9, 1),
                       "frac_of_hbm": round(whole / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                       "note": "gamma fused steps + confidence (h, W1 rows, w) + schedule "
                               "(survivals, SPS entries read, lengths) per step, over the "
                               "whole step's time"},
        "prewarm_ms": prewarm_ms,
        "cpu_baseline": None,
    }
    if not args.no_extras:
        # The same call with one weight copy (W2 stays in the Infinity Cache from
        # call to call), the other layout, and the three separate entry points.
        ms_h, d_h = run(args.path, args.layout, max(args.steps // 2, 1), max(args.warmup, 1),
                        ev_steps=20, copies=1)
        out["same_weights_every_step"] = dict(summary(ms_h, d_h), weight_copies=1,
                                              note="W2 found in the Infinity Cache by later calls")
        other = "tiled" if args.layout == "rgv" else "rgv"
        ms_o, d_o = run(args.path, other, max(args.steps // 2, 1), max(args.warmup, 1), ev_steps=20)
        out["other_layout"] = dict(summary(ms_o, d_o), layout=other)
        if args.path == "fused":
            ms_c, d_c = run("calls", args.layout, max(args.steps // 2, 1), max(args.warmup, 1),
                            ev_steps=20)
            out["three_calls"] = dict(summary(ms_c, d_c), launches_per_step=g + 4,
                                      call="dspark_markov_draft + dspark_confidence + dspark_schedule")
            ms_g = graph_steps(args.layout, max(args.steps // 2, 1), max(args.warmup, 1))
            out["graph_replay"] = {"ms_per_step": round(ms_g, 4),
                                   "value": round(R * g / (ms_g / 1e3), 1),
                                   "weight_copies": len(heads),
                                   "note": "the fused call captured in a HIP graph (one per "
                                           "weight copy) and replayed"}
        cold, cold_pos = cold_steps(args.layout, 10)
        out["cold"] = {"ms_per_step_median": round(cold, 4), "value": round(R * g / (cold / 1e3), 1),
                       "whole_step_frac_of_hbm": round(whole / (cold / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                       "fused_launch_us_by_position": cold_pos,
                       "frac_by_position": [round(nbytes / (u / 1e6) / 1e9 / HBM_PEAK_GBS, 4)
                                            for u in cold_pos],
                       "note": "a 512 MB read before each step (outside its events) evicts the "
                               "caches without leaving dirty lines to write back"}
        out["gemm_only"] = [gemm_only(args.config), gemm_only("long_block")]
        out["scheduler"] = scheduler_only()
        out["other_configs"] = [whole_step_config("qwen3_8b"), whole_step_config("long_block")]
        out["confidence"] = confidence_side()
        out["verify"] = verify_side()
        out["rnn_head"] = rnn_side()
        out["hbm_measured"] = hbm_measured()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
