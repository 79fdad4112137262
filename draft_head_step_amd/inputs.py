"""Seeded synthetic workloads for the Markov-head draft, confidence and prefix schedule.

This module only draws random numbers and packs them into the layouts the C-ABI
expects.  It holds none of the method's arithmetic, so both the CPU oracle's
tests and the GPU path can take their inputs from here.

Every tensor is drawn from its own ``numpy.random.Generator(PCG64)`` streams:
element chunks of 2^22 values each take the child seed (seed, tensor tag,
chunk index), so a workload is reproducible on any machine and independent of
how many threads fill it.  bf16 tensors are produced from float32 draws by
round-to-nearest-even and are returned as raw ``uint16`` bit patterns.

Layouts (row-major unless stated):
  W1       [V, r]     bf16  Markov embedding table; row t is W1[t].
  W2       [V, r]     bf16  the r x V logit projection stored column by column,
                            i.e. element (i, v) of W2 sits at v*r + i (the layout
                            of a linear layer's weight).
  base     [R, g, V]  fp32  backbone base logits; position k of request m is
                            base[m, k-1, :].
  h        [R, g, d]  bf16  backbone hidden states.
  w_conf   [d + r]    fp32  confidence weights, ordered [w_h; w_e].
  anchors  [R]        int32 anchor token of each request.
  uniforms [R, g, V]  fp32  open-interval uniforms for Gumbel-max sampling.
  sps      [B_max]    fp32  SPS lookup, sps[B-1] = SPS(B).
  conf     [R, g]     fp32  confidences (scheduler-only workload).

The synthetic distributions stand in for the trained DSpark weights, backbone
outputs and production traffic, none of which are available; their shapes
follow the drafters the DSpark pages describe (Qwen3 targets, DeepSeek-V4 with
Markov rank 512 and block size 5).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

GREEDY = 0
SAMPLE = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    R: int
    gamma: int
    V: int = 0
    r: int = 0
    d: int = 0
    mode: int = GREEDY
    temperature: float = 1.0
    w_std: float = 0.02          # std of W1 and W2 entries
    base_std: float = 2.0        # std of base logits
    boost_count: int = 0         # tokens per (request, position) raised by boost_value
    boost_value: float = 0.0
    h_std: float = 1.0
    wconf_std: float = 0.02
    sts: Optional[tuple] = None  # per-position confidence temperatures
    sps_kind: str = "staircase"  # "linear64" | "staircase"
    sps_bmax: int = 0            # 0 => R * (1 + gamma)
    beta_means: Optional[tuple] = None  # scheduler-only workload
    beta_conc: float = 8.0
    seed: int = 1

    @property
    def n_candidates(self) -> int:
        return self.R * self.gamma

    @property
    def b_max(self) -> int:
        return self.sps_bmax if self.sps_bmax else self.R * (1 + self.gamma)


CONFIGS = {
    # Correctness-sized workload.
    "tiny": Config("tiny", R=4, gamma=5, V=4096, r=64, d=256, w_std=0.02,
                   base_std=2.0, wconf_std=0.05, sps_kind="linear64", sps_bmax=64, seed=1),
    # Qwen3-8B-shaped drafter (V = 151936 is not a multiple of 256).
    "qwen3_8b": Config("qwen3_8b", R=64, gamma=5, V=151936, r=256, d=4096, base_std=3.0,
                       boost_count=8, boost_value=6.0, wconf_std=0.02,
                       sts=(1.0, 1.1, 1.2, 1.3, 1.4), seed=2),
    # DeepSeek-V4-shaped drafter, Markov rank 512, Gumbel-max sampling at T = 1.
    "dsv4": Config("dsv4", R=256, gamma=5, V=129280, r=512, d=7168, mode=SAMPLE,
                   temperature=1.0, base_std=3.0, wconf_std=0.02, seed=3),
    # Long block at high batch: 16 sequential steps re-reading a 66 MB W2.
    "long_block": Config("long_block", R=1024, gamma=16, V=129280, r=256, d=4096,
                         base_std=2.0, wconf_std=0.02, seed=4),
    # Scheduler stress: confidences given, staircase SPS over B = 1..65536.
    "sched_stress": Config("sched_stress", R=8192, gamma=7,
                           beta_means=(0.93, 0.89, 0.85, 0.82, 0.79, 0.76, 0.73),
                           beta_conc=8.0, sps_bmax=65536, seed=5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


CHUNK = 1 << 22
TAGS = {"W1": 1, "W2": 2, "base": 3, "boost": 4, "h": 5, "w_conf": 6, "anchors": 7,
        "uniforms": 8, "conf": 9, "v_tokens": 10, "v_target": 11, "v_match": 12,
        "v_draft_logits": 13, "v_noise": 14, "U_rnn": 15, "b_rnn": 16}


def _gen(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAGS[tag], idx])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(shape, dtype, seed: int, tag: str, draw) -> np.ndarray:
    """Fill an array chunk by chunk; chunk i comes from draw(generator(seed, tag, i), n)."""
    out = np.empty(shape, dtype=dtype)
    flat = out.reshape(-1)
    n = flat.size
    nch = (n + CHUNK - 1) // CHUNK

    def work(i):
        lo = i * CHUNK
        hi = min(n, lo + CHUNK)
        flat[lo:hi] = draw(_gen(seed, tag, i), hi - lo)

    if nch <= 1:
        for i in range(nch):
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out


def _normal_f32(std: float):
    def draw(g, n):
        x = g.standard_normal(size=n, dtype=np.float32)
        x *= np.float32(std)
        return x
    return draw


def _normal_bf16(seed, tag, shape, std: float) -> np.ndarray:
    nf = _normal_f32(std)
    return _fill(shape, np.uint16, seed, tag, lambda g, n: f32_to_bf16_bits(nf(g, n)))


def _open_uniform_draw(g, n):
    k = g.integers(0, 1 << 23, size=n, dtype=np.int32)
    u = k.astype(np.float32)
    u += np.float32(0.5)
    u *= np.float32(2.0 ** -23)
    return u


def open_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """u = (floor(U * 2^23) + 0.5) * 2^-23, exactly representable and inside [2^-24, 1 - 2^-24]."""
    n = int(np.prod(shape))
    return _open_uniform_draw(rng, n).reshape(shape)


def to_tiled(x: np.ndarray) -> np.ndarray:
    """[R, gamma, V] -> column-tiled [gamma, ceil(V/32), 32, R] (tail entries zero)."""
    R, g, V = x.shape
    C = (V + 31) // 32
    pad = np.zeros((R, g, C * 32), dtype=x.dtype)
    pad[:, :, :V] = x
    return np.ascontiguousarray(pad.reshape(R, g, C, 32).transpose(1, 2, 3, 0))


def from_tiled(t: np.ndarray, V: int) -> np.ndarray:
    """Column-tiled [gamma, C, 32, R] -> [R, gamma, V]."""
    g, C, _, R = t.shape
    return np.ascontiguousarray(t.transpose(3, 0, 1, 2).reshape(R, g, C * 32)[:, :, :V])


def sps_table(kind: str, b_max: int) -> np.ndarray:
    """Synthetic stand-ins for an engine's profiled steps-per-second curve, sps[B-1] = SPS(B)."""
    B = np.arange(1, b_max + 1, dtype=np.float64)
    if kind == "linear64":
        vals = (65.0 - B) / 64.0
    elif kind == "staircase":
        # plateaus of 512 tokens, each 3% below the previous one
        vals = 0.97 ** np.floor((B - 1.0) / 512.0)
    else:
        raise ValueError(kind)
    return vals.astype(np.float32)


def make_workload(cfg: Config, seed: Optional[int] = None, *, R: Optional[int] = None,
                  w_std: Optional[float] = None) -> dict:
    """Draw every input of one call of the path for ``cfg``.

    ``R`` overrides the request count (the leading requests of the full workload
    are not reproduced; the draw is a fresh, smaller workload).  ``w_std``
    overrides the std of W1/W2 (used for a bias-dominant variant of the tiny
    workload, where the Markov term actually moves the argmax).
    """
    seed = cfg.seed if seed is None else seed
    R = cfg.R if R is None else R
    g = cfg.gamma
    out = {"cfg": cfg, "R": R, "gamma": g, "seed": seed}
    b_max = cfg.sps_bmax if cfg.sps_bmax else R * (1 + g)
    b_max = max(b_max, R * (1 + g))
    if cfg.beta_means is not None:
        mu = np.asarray(cfg.beta_means, dtype=np.float64)
        a = cfg.beta_conc * mu
        b = cfg.beta_conc * (1.0 - mu)
        conf = _gen(seed, "conf").beta(a[None, :], b[None, :], size=(R, g)).astype(np.float32)
        out["conf"] = conf
        out["sps"] = sps_table(cfg.sps_kind, b_max)
        out["B_max"] = b_max
        return out
    V, r, d = cfg.V, cfg.r, cfg.d
    ws = cfg.w_std if w_std is None else w_std
    out.update(V=V, r=r, d=d, mode=cfg.mode, temperature=cfg.temperature)
    out["W1"] = _normal_bf16(seed, "W1", (V, r), ws)
    out["W2"] = _normal_bf16(seed, "W2", (V, r), ws)
    base = _fill((R, g, V), np.float32, seed, "base", _normal_f32(cfg.base_std))
    if cfg.boost_count:
        rng = _gen(seed, "boost")
        for m in range(R):
            for k in range(g):
                ids = rng.choice(V, size=cfg.boost_count, replace=False)
                base[m, k, ids] += np.float32(cfg.boost_value)
    out["base"] = base
    out["h"] = _normal_bf16(seed, "h", (R, g, d), cfg.h_std)
    out["w_conf"] = _normal_f32(cfg.wconf_std)(_gen(seed, "w_conf"), d + r)
    out["anchors"] = _gen(seed, "anchors").integers(0, V, size=(R,), dtype=np.int32)
    out["uniforms"] = (_fill((R, g, V), np.float32, seed, "uniforms", _open_uniform_draw)
                       if cfg.mode == SAMPLE else None)
    out["sts"] = None if cfg.sts is None else np.asarray(cfg.sts, dtype=np.float32)
    out["sps"] = sps_table(cfg.sps_kind, b_max)
    out["B_max"] = b_max
    return out


def make_head(cfg: Config, seed: Optional[int] = None, *, w_std: Optional[float] = None) -> dict:
    """W1, W2 and anchors of ``cfg`` only: the same streams as make_workload, so the
    arrays equal that workload's, without drawing the logits."""
    seed = cfg.seed if seed is None else seed
    ws = cfg.w_std if w_std is None else w_std
    V, r = cfg.V, cfg.r
    return {"W1": _normal_bf16(seed, "W1", (V, r), ws), "W2": _normal_bf16(seed, "W2", (V, r), ws),
            "anchors": _gen(seed, "anchors").integers(0, V, size=(cfg.R,), dtype=np.int32),
            "R": cfg.R, "gamma": cfg.gamma, "V": V, "r": r}


def make_rnn_head(cfg: Config, seed: Optional[int] = None, u_std: Optional[float] = None,
                  b_std: float = 0.5) -> dict:
    """Weights of the RNN head for cfg's sizes: U [2r, 2r + d] bf16 (rows: r gate
    units, then r candidate units; columns: the state, embedding and hidden
    blocks) ~ N(0, u_std) with u_std = 1/sqrt(2r + d) by default (pre-activations
    of order one), and b [2r] fp32 ~ N(0, b_std)."""
    seed = cfg.seed if seed is None else seed
    r, d = cfg.r, cfg.d
    std = (2 * r + d) ** -0.5 if u_std is None else u_std
    U = _normal_bf16(seed, "U_rnn", (2 * r, 2 * r + d), std)
    b = _normal_f32(b_std)(_gen(seed, "b_rnn"), 2 * r)
    return {"U": U, "b": b}


def make_verify_workload(R: int, gamma: int, V: int, seed: int = 11, match_rate: float = 0.7,
                         logit_std: float = 2.0) -> dict:
    """Inputs of the verification side: anchors, drafts, kept lengths, anchor
    positions, and target logits laid out per request and element,
    target[r, j] (j = 0..gamma) being the target's logits after element j of
    request r (its anchor, then draft j).  With probability match_rate the
    target's top token after element j is draft j + 1 (so drafts get accepted),
    else a random row.  The caller flattens target[r, :1 + l_r] in request order."""
    g = _gen(seed, "v_tokens")
    anchors = g.integers(0, V, size=R, dtype=np.int32)
    drafts = g.integers(0, V, size=(R, gamma), dtype=np.int32)
    lengths = g.integers(0, gamma + 1, size=R, dtype=np.int32)
    pos0 = g.integers(0, 4096, size=R, dtype=np.int32)
    target = _fill((R, 1 + gamma, V), np.float32, seed, "v_target", _normal_f32(logit_std))
    m = _gen(seed, "v_match").random(size=(R, gamma)) < match_rate
    for r in range(R):
        for j in range(gamma):
            if m[r, j]:
                target[r, j, drafts[r, j]] = target[r, j].max() + np.float32(1.0)
    return {"anchors": anchors, "tokens": drafts, "lengths": lengths, "pos0": pos0,
            "target": target, "R": R, "gamma": gamma, "V": V}


def make_accept_workload(n: int, V: int, seed: int = 12, draft_std: float = 3.0,
                         noise_std: float = 1.0) -> dict:
    """Paired draft / target logit rows [n, V]: target = draft + independent noise."""
    d = _fill((n, V), np.float32, seed, "v_draft_logits", _normal_f32(draft_std))
    t = d + _fill((n, V), np.float32, seed, "v_noise", _normal_f32(noise_std))
    return {"draft": d, "target": t}
