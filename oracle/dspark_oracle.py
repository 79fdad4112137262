"""CPU oracle for DSpark's Markov-head draft, confidence head and prefix scheduler.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP path.

It is deliberately plain: numpy arrays, float64 arithmetic wherever the pages
leave the precision open, one library primitive per step (a matmul, an argmax,
a stable sort, a cumulative sum) and no blocking, fusion or reordering.

Sources (the DSpark pages):
  [P1] "DSpark 深度解读" explainer (zhichai.net/topic/178208222):
       §二 设计一 -- semi-autoregressive generation, Markov-head equation;
       §二 设计二 -- Confidence Head equation, STS calibration,
                     Hardware-Aware Prefix Scheduler (objective and greedy steps);
       §三 挑战2 -- the early-stop break is removed in favour of a global search.
  [P3] DSpark news summary (10100.com/article/149061879), part 01 and Figure 1:
       the anchor is the first predicted position; Markov head default rank 256;
       prefix survival as the running product of conditional confidences.
  [P4] DeepSeek-V4-Pro DSpark integration note (demingchina.com/news/12928):
       markov_w1 / markov_w2 produce a logits bias, Markov rank 512, block
       size 5, fp32 confidences, greedy draft sampling.

Readings taken where the pages are silent or garbled (each one is also listed in
the design notes):
  * x_0 is the anchor; position k uses W1[x_{k-1}] ([P3] part 01).
  * Sampling is Gumbel-max with caller-supplied uniforms:
    x_k = argmax_v (z_v / T - ln(-ln u_v)).  Greedy is argmax_v z_v.
  * Argmax ties go to the smallest token id.
  * Confidence: c_k = sigmoid(s_k / T_k), s_k = w_h . h_k + w_e . W1[x_{k-1}],
    no bias term, w = [w_h; w_e] in fp32, one STS temperature per position
    (T_k = 1 when none is given).  c is rounded to fp32.
  * Survival a_{r,j} = prod_{i<=j} c_{r,i}, multiplied left to right in fp32.
  * B = sum_r (1 + l_r), tau = sum_r (1 + sum_{j<=l_r} a_{r,j}) -- the "1 +" is
    the anchor/bonus token every request verifies.
  * tau is accumulated in fixed point: q = rint(a * 2^40) as an unsigned 64-bit
    integer, so the sum is exact and independent of summation order; Theta is
    the fp64 product double(R*2^40 + S_m) * 2^-40 * double(SPS(R+m)).
  * The argmax over the budget takes the smallest B on ties; candidates with
    equal survival are ordered by (request, position).
  * The scheduler clamps survivals into [0, 1] (NaN taken as 0): they are
    probabilities, and the clamp keeps the fixed-point tau below 2^64.
"""
from __future__ import annotations

import numpy as np

GREEDY = 0
SAMPLE = 1
TAU_FRAC_BITS = 40
TAU_SCALE = float(1 << TAU_FRAC_BITS)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float64: a bf16 value is the top half of an fp32 word."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def w2_matrix(W2_store: np.ndarray) -> np.ndarray:
    """The r x V matrix W2 from its [V, r] storage (element (i, v) at v*r + i)."""
    return bf16_to_f64(W2_store).T


# ---------------------------------------------------------------------------
# Markov head -- [P1] §二 设计一, Markov-head equation; [P3] part 01; [P4] config
# ---------------------------------------------------------------------------

def markov_bias(W1: np.ndarray, W2_store: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """B(x_{k-1}, .) = W1[x_{k-1}] W2 for every request: [n] token ids -> [n, V] fp64."""
    e = bf16_to_f64(W1[np.asarray(prev, dtype=np.int64)])      # [n, r]
    return e @ w2_matrix(W2_store)                              # [n, r] x [r, V]


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel noise from open-interval uniforms: -ln(-ln u), fp64."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))


def select(z: np.ndarray, mode: int, temperature: float = 1.0, u: np.ndarray | None = None):
    """Pick the draft token of each row of z ([n, V], fp64).

    Greedy: argmax_v z_v.  Sample: argmax_v (z_v / T + g_v) with g = -ln(-ln u).
    Returns (token ids [n], scores that were maximised [n, V], margin [n]) where
    margin = top-1 minus top-2 score of the row.
    """
    if mode == GREEDY:
        s = z
    elif mode == SAMPLE:
        if u is None:
            raise ValueError("sampling needs uniforms")
        s = z / float(temperature) + gumbel(u)
    else:
        raise ValueError(f"unknown mode {mode}")
    x = np.argmax(s, axis=1)                         # first index among equal maxima
    if s.shape[1] >= 2:
        top2 = np.partition(s, s.shape[1] - 2, axis=1)[:, -2:]
        margin = top2[:, 1] - top2[:, 0]
    else:
        margin = np.full(s.shape[0], np.inf)
    return x.astype(np.int32), s, margin


def markov_draft(W1, W2_store, base, anchors, mode=GREEDY, temperature=1.0, uniforms=None,
                 prev_tokens=None, rows=None, keep_bias=False):
    """The gamma-step sequential refinement z_k = base_k + W1[x_{k-1}] W2, x_0 = anchor.

    ``prev_tokens`` ([R, gamma], optional) replays the chain with another
    implementation's tokens as the previous-token inputs, so that each step can
    be checked on its own ("forced sequence").  ``rows`` restricts the work to a
    subset of requests.

    Returns dict with tokens [n, gamma] int32, margin [n, gamma] fp64,
    and (if keep_bias) bias [n, gamma, V] fp64.
    """
    R, g, V = base.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.size
    tokens = np.zeros((n, g), dtype=np.int32)
    margin = np.zeros((n, g), dtype=np.float64)
    bias_all = np.zeros((n, g, V), dtype=np.float64) if keep_bias else None
    prev = np.asarray(anchors, dtype=np.int64)[rows]
    for k in range(g):
        bias = markov_bias(W1, W2_store, prev)
        z = base[rows, k, :].astype(np.float64) + bias
        u = None if uniforms is None else uniforms[rows, k, :]
        x, _, mg = select(z, mode, temperature, u)
        tokens[:, k] = x
        margin[:, k] = mg
        if keep_bias:
            bias_all[:, k, :] = bias
        prev = x.astype(np.int64) if prev_tokens is None else \
            np.asarray(prev_tokens, dtype=np.int64)[rows, k]
    out = {"tokens": tokens, "margin": margin}
    if keep_bias:
        out["bias"] = bias_all
    return out


def step_scores(W1, W2_store, base_k, prev, mode=GREEDY, temperature=1.0, u_k=None):
    """One step on its own: scores s ([n, V] fp64), argmax ids and margins for given x_{k-1}."""
    z = base_k.astype(np.float64) + markov_bias(W1, W2_store, prev)
    x, s, mg = select(z, mode, temperature, u_k)
    return x, s, mg


# ---------------------------------------------------------------------------
# RNN head -- [P3] part 01 (the second, lightweight sequential stage: a recurrent
# in-block state, updated by a gate over the concatenation of the history
# state, the previous token's embedding and the backbone hidden state);
# [P1] §二 设计一 (the RNN head keeps a recurrent state that remembers the whole
# prefix).  The pages give no equations; the reading taken here:
#   u_k   = [s_{k-1}; e_k; h_k],  e_k = W1[x_{k-1}] (x_0 = anchor), s_0 = 0
#   g_k   = sigmoid(G u_k + b_g)                 (update gate, r units)
#   c_k   = e_k + tanh(C u_k + b_c)              (candidate: the embedding row
#                                                 plus a correction)
#   s_k   = g_k * c_k + (1 - g_k) * s_{k-1}
#   z_k   = base_k + s_k W2                      (the same low-rank projection
#                                                 to the vocabulary as the Markov head)
# G and C are stored stacked as U [2r, 2r + d] (rows: the r gate units, then the
# r candidate units; columns: the s, e and h blocks), b = [b_g; b_c] [2r].
# Products take bf16 operands (weights, h and e are bf16; the state, kept in
# higher precision, is rounded to bf16 where it enters a product: fp32 first,
# then bf16, each to nearest even).  A saturated gate (g = 1) with C = 0 and
# b_c = 0 gives s_k = e_k: the Markov head.
# ---------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Value of x rounded to fp32 and then to bf16 (both to nearest, ties to even),
    as float64."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    keep = ((u >> 16) & 1) + 0x7FFF
    top = ((u + keep) >> 16) << 16
    finite = np.isfinite(x32)
    out = np.where(finite, top, u & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32).astype(np.float64)


def rnn_update(s_prev, e, h_k, U, b):
    """One gated update of the recurrent state: [n, r] states, [n, r] embedding
    rows (fp64 values of bf16), [n, d] hidden states -> new states [n, r] fp64."""
    r = e.shape[1]
    Uf = bf16_to_f64(U)                                   # [2r, 2r + d]
    u = np.concatenate([bf16_round(s_prev), e, h_k], axis=1)
    pre = u @ Uf.T + np.asarray(b, dtype=np.float64)[None, :]
    g = sigmoid(pre[:, :r])
    cand = e + np.tanh(pre[:, r:])
    return g * cand + (1.0 - g) * s_prev


def rnn_draft(W1, W2_store, U, b, base, h, anchors, mode=GREEDY, temperature=1.0,
              uniforms=None, prev_tokens=None, rows=None, keep_state=False, keep_scores=False):
    """The gamma-step RNN-head refinement (reading above).  ``prev_tokens`` replays
    the chain with another implementation's tokens as the previous-token inputs
    (the state then evolves from those tokens), as in markov_draft.

    Returns dict with tokens [n, gamma], margin [n, gamma], and optionally the
    states [n, gamma, r] (fp64) and the maximised scores [n, gamma, V]."""
    R, g, V = base.shape
    r = W1.shape[1]
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.size
    tokens = np.zeros((n, g), dtype=np.int32)
    margin = np.zeros((n, g), dtype=np.float64)
    states = np.zeros((n, g, r)) if keep_state else None
    scores = np.zeros((n, g, V)) if keep_scores else None
    prev = np.asarray(anchors, dtype=np.int64)[rows]
    s = np.zeros((n, r), dtype=np.float64)
    W2m = w2_matrix(W2_store)
    for k in range(g):
        e = bf16_to_f64(W1[prev])
        s = rnn_update(s, e, bf16_to_f64(h[rows, k, :]), U, b)
        z = base[rows, k, :].astype(np.float64) + bf16_round(s) @ W2m
        u = None if uniforms is None else uniforms[rows, k, :]
        x, sc, mg = select(z, mode, temperature, u)
        tokens[:, k] = x
        margin[:, k] = mg
        if keep_state:
            states[:, k, :] = s
        if keep_scores:
            scores[:, k, :] = sc
        prev = x.astype(np.int64) if prev_tokens is None else \
            np.asarray(prev_tokens, dtype=np.int64)[rows, k]
    out = {"tokens": tokens, "margin": margin}
    if keep_state:
        out["states"] = states
    if keep_scores:
        out["scores"] = scores
    return out


# ---------------------------------------------------------------------------
# Confidence head and STS -- [P1] §二 设计二 (Confidence Head, STS); [P4] fp32 output
# ---------------------------------------------------------------------------

def sigmoid(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def confidence_logits(h, W1, anchors, tokens, w_conf):
    """s_{m,k} = w_h . h_{m,k} + w_e . W1[x_{k-1}] in fp64: [R, gamma]."""
    R, g, d = h.shape
    w = np.asarray(w_conf, dtype=np.float64)
    w_h, w_e = w[:d], w[d:]
    s = np.zeros((R, g), dtype=np.float64)
    prev = np.asarray(anchors, dtype=np.int64)
    for k in range(g):
        e = bf16_to_f64(W1[prev])
        s[:, k] = bf16_to_f64(h[:, k, :]) @ w_h + e @ w_e
        prev = np.asarray(tokens, dtype=np.int64)[:, k]
    return s


def confidence(h, W1, anchors, tokens, w_conf, sts_temp=None):
    """c_{m,k} = fl32(sigmoid(s_{m,k} / T_k)), T_k from STS (1 if none): [R, gamma] fp32."""
    s = confidence_logits(h, W1, anchors, tokens, w_conf)
    g = s.shape[1]
    T = np.ones(g) if sts_temp is None else np.asarray(sts_temp, dtype=np.float64)
    return sigmoid(s / T[None, :]).astype(np.float32)


# ---------------------------------------------------------------------------
# Prefix survival -- [P1] §二 设计二, scheduler definitions; [P3] part 01
# ---------------------------------------------------------------------------

def survival(conf: np.ndarray) -> np.ndarray:
    """a_{r,1} = c_{r,1}; a_{r,j} = fl32(a_{r,j-1} * c_{r,j}), left to right."""
    c = np.asarray(conf, dtype=np.float32)
    a = np.empty_like(c)
    a[:, 0] = c[:, 0]
    for j in range(1, c.shape[1]):
        a[:, j] = a[:, j - 1] * c[:, j]          # fp32 * fp32 -> fp32, round to nearest even
    return a


# ---------------------------------------------------------------------------
# Hardware-aware prefix scheduler -- [P1] §二 设计二 (objective, greedy steps 1-4),
# §三 挑战2 (no early stop: global search over every budget); [P3] part 01
# ---------------------------------------------------------------------------

def clamp_survival(surv: np.ndarray) -> np.ndarray:
    """Survivals are probabilities: values outside [0, 1] are clamped into it and
    NaN is taken as 0, before the sort and the fixed-point sums."""
    a = np.asarray(surv, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        return np.where(a > 0, np.minimum(a, np.float32(1.0)), np.float32(0.0)).astype(np.float32)


def candidate_order(surv: np.ndarray) -> np.ndarray:
    """Candidate ids r*gamma + (j-1) sorted by survival descending, ties by id ascending."""
    key = clamp_survival(surv).reshape(-1)
    return np.argsort(-key, kind="stable").astype(np.int32)


def schedule(surv: np.ndarray, sps: np.ndarray):
    """Maximise Theta = tau * SPS(B) over every B in [R, R(1+gamma)].

    Returns dict: lengths [R] int32, order [R*gamma] int32, m_star, B_star,
    tau_fx (uint64 fixed point), tau (fp64), theta (fp64), theta_all [N+1].
    """
    a = clamp_survival(surv)
    R, g = a.shape
    N = R * g
    sps = np.asarray(sps, dtype=np.float32)
    if sps.size < R * (1 + g):
        raise ValueError("SPS table must cover B up to R * (1 + gamma)")
    order = candidate_order(a)
    q = np.rint(a.reshape(-1).astype(np.float64) * TAU_SCALE).astype(np.uint64)
    S = np.zeros(N + 1, dtype=np.uint64)
    S[1:] = np.cumsum(q[order], dtype=np.uint64)
    tau_fx = np.uint64(R) * np.uint64(1 << TAU_FRAC_BITS) + S
    tau = tau_fx.astype(np.float64) * (1.0 / TAU_SCALE)
    B = R + np.arange(N + 1)
    theta = tau * sps[B - 1].astype(np.float64)
    m_star = int(np.argmax(theta))                       # smallest m (= smallest B) on ties
    lengths = np.bincount(order[:m_star] // g, minlength=R).astype(np.int32)
    return {"lengths": lengths, "order": order, "m_star": m_star, "B_star": R + m_star,
            "tau_fx": int(tau_fx[m_star]), "tau": float(tau[m_star]),
            "theta": float(theta[m_star]), "theta_all": theta}


def _tau_fx_prefix(a: np.ndarray, order: np.ndarray, m: int) -> int:
    """R * 2^40 + sum of the fixed-point survivals of the first m sorted candidates."""
    R = a.shape[0]
    q = np.rint(a.reshape(-1).astype(np.float64) * TAU_SCALE).astype(np.uint64)
    return int(R) * (1 << TAU_FRAC_BITS) + int(np.sum(q[order[:m]], dtype=np.uint64))


def _result(a: np.ndarray, order: np.ndarray, m: int, theta: float):
    R, g = a.shape
    tau_fx = _tau_fx_prefix(a, order, m)
    lengths = np.bincount(order[:m] // g, minlength=R).astype(np.int32)
    return {"lengths": lengths, "order": order, "m_star": m, "B_star": R + m,
            "tau_fx": tau_fx, "tau": float(np.float64(tau_fx) * (1.0 / TAU_SCALE)),
            "theta": theta}


def schedule_early_stop(surv: np.ndarray, sps: np.ndarray):
    """The greedy scheduler with its early-stop break ([P1] §二 设计二, greedy steps
    3-5; [P3] part 01, the theoretical version): admit candidates one at a time in
    the sorted order, look Theta up after each admission, and stop as soon as Theta
    no longer increases (Theta_m <= Theta_{m-1}: the m-th candidate is not
    admitted).  Theta_m is computed exactly as in schedule().  Sequential on purpose."""
    a = clamp_survival(surv)
    R, g = a.shape
    N = R * g
    sps = np.asarray(sps, dtype=np.float32)
    if sps.size < R * (1 + g):
        raise ValueError("SPS table must cover B up to R * (1 + gamma)")
    order = candidate_order(a)
    flat = a.reshape(-1)
    tau_fx = int(R) * (1 << TAU_FRAC_BITS)

    def theta_of(fx, m):
        return float(np.float64(fx) * (1.0 / TAU_SCALE)) * float(np.float64(sps[R + m - 1]))

    best = theta_of(tau_fx, 0)
    m = 0
    while m < N:
        fx = tau_fx + int(np.rint(np.float64(flat[order[m]]) * TAU_SCALE))
        th = theta_of(fx, m + 1)
        if not th > best:
            break
        tau_fx, best, m = fx, th, m + 1
    return _result(a, order, m, best)


def schedule_capacity(surv: np.ndarray, capacity: int):
    """Capacity-K schedule ([P1] §三 挑战1; [P3] part 01, the asynchronous
    production form): a verification batch of `capacity` tokens, predicted two
    steps earlier, is filled with the anchors plus the top candidates by current
    survival: m* = clamp(K - R, 0, R * gamma) in the sorted order of schedule().
    There is no SPS table here; Theta is reported as tau*."""
    a = clamp_survival(surv)
    R, g = a.shape
    order = candidate_order(a)
    m = min(max(int(capacity) - R, 0), R * g)
    tau = float(np.float64(_tau_fx_prefix(a, order, m)) * (1.0 / TAU_SCALE))
    return _result(a, order, m, tau)


# ---------------------------------------------------------------------------
# Verification side -- [P1] §三 挑战3 (every verified token is one flattened
# element; a marker tensor carries the within-sequence dependencies); [P3]
# Figure 1 (the target verifies anchor + kept prefix in parallel, accepts the
# matching prefix and emits a corrected token); [P1] §二 设计二 (the acceptance
# label 1 - TV(p^d, p^t)).
# ---------------------------------------------------------------------------

def verify_pack(anchors, tokens, lengths, pos0=None):
    """Flatten the scheduled prefixes: request r contributes 1 + l_r elements,
    its anchor then its first l_r drafts, at positions pos0[r] + j (pos0 = 0 if
    not given), each marked with r.  cu_seqlens[r] is where request r starts;
    cu_seqlens[R] = B = sum_r (1 + l_r)."""
    anchors = np.asarray(anchors, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    R, g = tokens.shape
    lengths = np.asarray(lengths, dtype=np.int64)
    pos0 = np.zeros(R, np.int64) if pos0 is None else np.asarray(pos0, dtype=np.int64)
    cu = np.zeros(R + 1, np.int64)
    flat_tok, flat_pos, flat_req = [], [], []
    for r in range(R):
        n = 1 + int(lengths[r])
        cu[r + 1] = cu[r] + n
        for j in range(n):
            flat_tok.append(int(anchors[r]) if j == 0 else int(tokens[r, j - 1]))
            flat_pos.append(int(pos0[r]) + j)
            flat_req.append(r)
    return {"tokens": np.array(flat_tok, np.int32), "positions": np.array(flat_pos, np.int32),
            "request": np.array(flat_req, np.int32), "cu_seqlens": cu.astype(np.int32),
            "B": int(cu[R])}


def verify_greedy(target_logits, cu_seqlens, tokens, lengths):
    """Greedy verification of the flattened batch: t = argmax of each target row
    (the target's next token after that element; ties -> smallest id).  For
    request r starting at s = cu_seqlens[r], draft j (1-based) is accepted while
    tokens[r, j-1] == t[s + j - 1] for every earlier j; a = the number accepted
    (<= l_r); the next token is t[s + a] -- the correction of the first rejected
    draft, or the bonus token when all l_r are accepted."""
    t = np.argmax(np.asarray(target_logits, dtype=np.float32), axis=1).astype(np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    R = tokens.shape[0]
    accepted = np.zeros(R, np.int32)
    nxt = np.zeros(R, np.int32)
    for r in range(R):
        s = int(cu_seqlens[r])
        a = 0
        while a < int(lengths[r]) and tokens[r, a] == t[s + a]:
            a += 1
        accepted[r] = a
        nxt[r] = t[s + a]
    return {"target_argmax": t.astype(np.int32), "accepted": accepted, "next_token": nxt}


def softmax64(z: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    x = np.asarray(z, dtype=np.float64) / float(temperature)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def accept_prob(draft_logits, target_logits, temperature: float = 1.0):
    """Per row: sum_v min(p^d_v, p^t_v) with p = softmax(logits / T) -- the
    probability that a token drawn from the draft distribution survives the
    rejection test against the target, which equals 1 - TV(p^d, p^t), the
    confidence head's training label."""
    p = softmax64(draft_logits, temperature)
    q = softmax64(target_logits, temperature)
    return np.minimum(p, q).sum(axis=-1)


def run_path(wl: dict, rows=None):
    """Draft -> confidence -> survival -> schedule for one workload (the whole hot path)."""
    dr = markov_draft(wl["W1"], wl["W2"], wl["base"], wl["anchors"], wl["mode"],
                      wl["temperature"], wl["uniforms"], rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    c = confidence(wl["h"][sel], wl["W1"], np.asarray(wl["anchors"])[sel], dr["tokens"],
                   wl["w_conf"], wl["sts"])
    a = survival(c)
    sc = schedule(a, wl["sps"])
    return {"draft": dr, "conf": c, "surv": a, "schedule": sc}
