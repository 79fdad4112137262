/*
 * dspark.h -- C ABI of the DSpark drafter hot path on AMD Instinct MI355X (gfx950).
 *
 * The path: a gamma-step Markov-head refinement of a parallel backbone's base
 * logits, the confidence head with per-position temperature calibration, the
 * prefix survival products, and the hardware-aware prefix scheduler that picks
 * per-request verification lengths maximising tau * SPS(B).
 *
 * Sources (the DSpark pages):
 *   [P1] DSpark explainer (zhichai.net/topic/178208222): section 二 "design 1"
 *        (Markov-head equation), section 二 "design 2" (confidence head, STS,
 *        hardware-aware prefix scheduler), section 三 challenges 1-2 (asynchronous
 *        top-K scheduling, global search without early stop).
 *   [P3] DSpark news summary (10100.com/article/149061879), part 01 and Figure 1
 *        (anchor as first predicted position, Markov rank 256, survival products).
 *   [P4] DeepSeek-V4-Pro DSpark integration note (demingchina.com/news/12928)
 *        (markov_w1/markov_w2 logits bias, rank 512, block size 5, fp32
 *        confidences, greedy draft sampling).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers into caller-owned memory on the
 *     current HIP device, row-major, densely packed.  bf16 tensors are passed
 *     as raw 16-bit patterns (uint16_t).  The library keeps no pointer after
 *     the call returns and allocates no device memory: scratch comes from a
 *     caller-provided workspace whose size the *_workspace() queries return.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising the host, so calls can be
 *     captured in HIP graphs.  Calls on different streams with distinct
 *     outputs and workspaces may run concurrently.
 *   - Host-visible argument checks run before anything is enqueued; a failing
 *     check returns a status other than DSPARK_OK and enqueues nothing.  Token
 *     ids inside device buffers (anchors, tokens) are checked on the device:
 *     the draft turns a request whose anchor lies outside [0, V) into tokens
 *     of -1, and the confidence head gives NaN for a position whose previous
 *     token lies outside [0, V), so a bad id is detectable rather than
 *     silently clamped.
 *   - dspark_last_error() returns a thread-local description of the last
 *     failure on the calling thread.
 *
 * Notation: R requests, gamma draft positions per request, V vocabulary size,
 * r Markov rank, d backbone hidden size.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,       /* NULL required pointer, non-positive size, bad mode or temperature */
  DSPARK_EWORKSPACE = 2,   /* workspace NULL or smaller than the query says */
  DSPARK_EUNSUPPORTED = 3, /* valid but outside what the kernels are built for (see each call) */
  DSPARK_EDEVICE = 4       /* a HIP launch or runtime call failed; see dspark_last_error() */
} dspark_status;

typedef enum {
  DSPARK_GREEDY = 0, /* x_k = argmax_v z_v */
  DSPARK_SAMPLE = 1  /* x_k = argmax_v (z_v / T - ln(-ln u_v))  (Gumbel-max) */
} dspark_mode;

/* Storage order of the [R, gamma, V] fp32 arrays of dspark_markov_draft (base,
 * uniforms, bias_out).  Element (m, k, v) -- request m, position k (0-based),
 * vocabulary entry v -- sits at
 *   DSPARK_LAYOUT_RGV:   (m * gamma + k) * V + v                     (row-major [R][gamma][V])
 *   DSPARK_LAYOUT_TILED: ((k * C + v / 32) * 32 + v % 32) * R + m,  C = ceil(V / 32)
 * The tiled order ([gamma][C][32][R], the tail entries of the last chunk
 * padding) is column-major inside each 32-entry chunk: for one vocabulary
 * entry the requests are contiguous, so every load of a 32-request tile reads
 * whole 128-byte lines and a chunk of all requests is one contiguous block
 * (the logits-transposed output of a backbone LM-head GEMM, or a random-number
 * fill, produces it at no extra cost).  Row-major arrays are read with the
 * vocabulary entries on the lanes instead, so there a load reads 128
 * contiguous bytes of one request row. */
typedef enum {
  DSPARK_LAYOUT_RGV = 0,
  DSPARK_LAYOUT_TILED = 1
} dspark_layout;

/* Limits of this build. */
#define DSPARK_MAX_RANK 512          /* r <= 512 and r % 16 == 0 */
#define DSPARK_MAX_CANDIDATES (1 << 23) /* R * gamma; also R * (1 + gamma) < 2^24, which keeps
                                           the fixed-point tau sum exact (below 2^64) */

/* Optional per-step timing hooks for dspark_markov_draft.  When non-NULL,
 * begin[k] and end[k] (k = 0..gamma-1) receive the start and stop time of the
 * fused step kernel of position k+1: they are attached to that kernel's
 * dispatch (hipExtLaunchKernel), so hipEventElapsedTime(begin[k], end[k]) is
 * the kernel's own duration.  Each entry is a hipEvent_t created by the caller
 * (NULL entries are skipped); count must be >= gamma. */
typedef struct {
  void* const* begin;
  void* const* end;
  int count;
} dspark_step_events;

/* Result summary of dspark_schedule, written to DEVICE memory (32 bytes). */
typedef struct {
  int32_t B_star;   /* chosen verification budget B* = R + m* */
  int32_t m_star;   /* number of draft tokens admitted, summed over requests */
  uint64_t tau_fx;  /* tau* in fixed point, units of 2^-40 */
  double tau;       /* tau* = tau_fx * 2^-40 (double rounding of tau_fx, then exact scale) */
  double theta;     /* Theta* = tau * SPS(B*) */
} dspark_schedule_info;

/* Bytes of workspace dspark_markov_draft needs for these sizes (0 if invalid). */
size_t dspark_markov_draft_workspace(int R, int gamma, int V, int r);

/*
 * Markov-head draft: the gamma sequential refinement steps of [P1] section 二
 * design 1 (Markov-head equation B(x_{k-1}, .) = W1[x_{k-1}] W2), with x_0 the
 * anchor ([P3] part 01) and the logits bias added to the backbone's base
 * logits ([P4]).  For k = 1..gamma and every request m:
 *     e      = W1[x_{k-1}, :]                         (r values)
 *     z_v    = base[m, k-1, v] + sum_i e_i * W2(i, v)  (fp32, bf16 products, fp32 accumulation)
 *     x_k    = argmax_v z_v                            (GREEDY)
 *            = argmax_v z_v / T - ln(-ln u[m,k-1,v])   (SAMPLE)
 * Equal maxima resolve to the smallest token id.
 *
 *   W1        [V, r] bf16   Markov embedding table (row t = W1[t]).
 *   W2        [V, r] bf16   the r x V projection stored column by column:
 *                           element (i, v) at W2[v * r + i].
 *   layout    DSPARK_LAYOUT_RGV or DSPARK_LAYOUT_TILED: storage order of base,
 *             uniforms and bias_out (see dspark_layout).
 *   base      [R, gamma, V] fp32 backbone base logits (in `layout` order; the
 *             tiled order holds gamma * C * 32 * R floats).  NULL in GREEDY mode
 *             drafts from the Markov bias alone (base taken as zero; no logits
 *             are read, so a call costs the gather + bias GEMM + argmax only).
 *   anchors   [R] int32     anchor token of each request (x_0); a request whose
 *                           anchor is outside [0, V) gets tokens -1 throughout.
 *   mode      DSPARK_GREEDY or DSPARK_SAMPLE.
 *   temperature  > 0 and finite when mode == DSPARK_SAMPLE; ignored for GREEDY.
 *   uniforms  [R, gamma, V] fp32 in (0, 1) in `layout` order, required iff SAMPLE
 *             (NULL for GREEDY).
 *   tokens    [R, gamma] int32 output, tokens[m * gamma + k - 1] = x_k (-1 after a
 *             bad anchor, or where every score of a row is -inf or NaN).
 *   bias_out  optional [R, gamma, V] fp32 output (in `layout` order) of the
 *             Markov bias of every step (a debugging aid; NULL on the hot path).
 *   workspace device scratch of ws_bytes >= dspark_markov_draft_workspace(...),
 *             16-byte aligned: up to 16 packed 64-bit partial results per
 *             request and step.  Its contents on entry do not matter (the call clears what
 *             it uses in its first launch).
 *   events    optional timing hooks (NULL on the hot path).
 * Errors: EINVAL for NULL required pointers (base is optional only in GREEDY
 * mode), W1 or W2 not 16-byte aligned, R/gamma/V/r <= 0, V < 2, a bad layout
 * or mode, a non-positive or non-finite temperature in SAMPLE mode, or
 * uniforms given in GREEDY mode; EUNSUPPORTED for r > DSPARK_MAX_RANK or
 * r % 16 != 0, and where the 32-bit byte offsets of one step would overflow:
 * ceil(V/32)*32*r > 2^30, gamma*V >= 2^22 (DSPARK_LAYOUT_RGV, per block of
 * requests) or ceil(V/32)*R >= 2^24 (DSPARK_LAYOUT_TILED, all requests); EWORKSPACE if the workspace
 * is NULL or too small, EINVAL if it is not 16-byte aligned; EDEVICE on a
 * launch failure.
 */
dspark_status dspark_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int layout, int mode, float temperature, const float* uniforms,
                                  int32_t* tokens, float* bias_out, void* workspace,
                                  size_t ws_bytes, const dspark_step_events* events,
                                  void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * draft as dspark_markov_draft with no bias output, no timing hooks and no
 * workspace argument.  Its scratch (the packed per-step results) lives in a
 * static device array of DSPARK_NOALLOC_SCRATCH_BYTES that each GPU holds
 * until the process ends; the call allocates nothing.
 * Limit: dspark_markov_draft_workspace(R, gamma, V, r) <= DSPARK_NOALLOC_SCRATCH_BYTES,
 * i.e. R * gamma <= 32768; larger sizes return DSPARK_EUNSUPPORTED.
 * Concurrency: every call on one GPU uses that GPU's one array, so calls that
 * overlap in time on the same device (other streams, other host threads) race
 * and must be serialised by the caller.  Each call clears what it uses first.
 * Errors: as dspark_markov_draft (without the workspace errors), plus
 * EUNSUPPORTED above the limit and EDEVICE if the array's address cannot be
 * found on the current device.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES (4u << 20)
dspark_status dspark_markov_draft_noalloc(const uint16_t* W1, const uint16_t* W2,
                                          const float* base, const int32_t* anchors, int R,
                                          int gamma, int V, int r, int layout, int mode,
                                          float temperature, const float* uniforms,
                                          int32_t* tokens, void* stream);

/* Bytes of workspace dspark_rnn_draft needs (0 if invalid). */
size_t dspark_rnn_draft_workspace(int R, int gamma, int V, int r, int d);

/*
 * RNN-head draft: the alternative sequential stage of [P3] part 01 (a
 * recurrent in-block state updated by a gate over the concatenated history
 * state, previous-token embedding and backbone hidden state; [P1] section 二
 * design 1, the RNN head that remembers the whole prefix).  The pages give no
 * equations; this build reads them as, for k = 1..gamma and every request m,
 *     u_k = [s_{k-1}; e_k; h_k],  e_k = W1[x_{k-1}, :] (x_0 = anchor),  s_0 = 0
 *     g_k = sigmoid(G u_k + b_g)             (update gate, r units)
 *     c_k = e_k + tanh(C u_k + b_c)          (candidate: embedding row + correction)
 *     s_k = g_k * c_k + (1 - g_k) * s_{k-1}  (fp32 state)
 *     z_v = base[m, k-1, v] + sum_i bf16(s_k)_i W2(i, v),  x_k selected as in
 *           dspark_markov_draft (GREEDY or SAMPLE)
 * Products take bf16 operands with fp32 accumulation: the state enters them
 * rounded to bf16.  A gate saturated at 1 with C = 0, b_c = 0 is the Markov head.
 *   U         [2r, 2r + d] bf16, 16-byte aligned: rows 0..r-1 are G, rows
 *             r..2r-1 are C; columns [0, r) act on s_{k-1}, [r, 2r) on e_k,
 *             [2r, 2r + d) on h_k.
 *   b_rnn     [2r] fp32 = [b_g; b_c].
 *   h         [R, gamma, d] bf16 backbone hidden states (16-byte aligned), d % 8 == 0.
 *   W1, W2, base, anchors, layout, mode, temperature, uniforms, tokens, events
 *             as for dspark_markov_draft (no bias output).
 *   state_out optional [R, r] fp32 output: the state s_gamma after the last step
 *             (a debugging aid; NULL on the hot path).
 *   workspace >= dspark_rnn_draft_workspace(R, gamma, V, r, d) bytes, 256-byte
 *             aligned: packed words, the token-independent pre-activations and
 *             two copies of the state.
 * A call is 2 gamma + 2 launches.  Errors: as dspark_markov_draft, plus EINVAL
 * for NULL U / b_rnn / h or d <= 0, EUNSUPPORTED for d % 8 != 0, a misaligned U
 * or h, R * gamma * 2r >= 2^31, or 2r + d > 2^22.
 */
dspark_status dspark_rnn_draft(const uint16_t* W1, const uint16_t* W2, const uint16_t* U,
                               const float* b_rnn, const float* base, const uint16_t* h,
                               const int32_t* anchors, int R, int gamma, int V, int r, int d,
                               int layout, int mode, float temperature, const float* uniforms,
                               int32_t* tokens, float* state_out, void* workspace, size_t ws_bytes,
                               const dspark_step_events* events, void* stream);

/*
 * Confidence head with STS calibration, [P1] section 二 design 2 (confidence
 * head equation, sequential temperature scaling) and [P4] (fp32 scores):
 *     s_{m,k} = sum_{i<d} w[i] h[m,k-1,i] + sum_{i<r} w[d+i] W1[x_{k-1}, i]
 *     c_{m,k} = 1 / (1 + exp(-s_{m,k} / T_k))
 * with x_0 = anchors[m] and x_k = tokens[m, k-1].  Optionally also the prefix
 * survival a_{m,j} = c_{m,1} * ... * c_{m,j}, multiplied left to right in fp32.
 *
 *   h         [R, gamma, d] bf16 backbone hidden states.
 *   W1        [V, r] bf16 (as in dspark_markov_draft).
 *   anchors   [R] int32; tokens [R, gamma] int32 (the draft).
 *   w_conf    [d + r] fp32, ordered [w_h; w_e].
 *   sts_temp  optional [gamma] fp32 positive temperatures T_k (NULL => 1).
 *   conf      [R, gamma] fp32 output c.
 *   surv      optional [R, gamma] fp32 output a (NULL to skip).
 * Errors: EINVAL for NULL required pointers or non-positive sizes; EDEVICE on a
 * launch failure.  Temperatures are device data: they must be positive.  A
 * position whose x_{k-1} lies outside [0, V) gets c = NaN (and so do its
 * survival and the later ones of that request).
 */
dspark_status dspark_confidence(const uint16_t* h, const uint16_t* W1, const int32_t* anchors,
                                const int32_t* tokens, const float* w_conf,
                                const float* sts_temp, int R, int gamma, int d, int V, int r,
                                float* conf, float* surv, void* stream);

/*
 * Prefix survival alone ([P1] section 二 design 2, scheduler definitions):
 * surv[m, j] = conf[m, 0] * ... * conf[m, j], sequential fp32 products.
 * conf and surv are [R, gamma] fp32 device arrays (they may not alias).
 */
dspark_status dspark_survival(const float* conf, int R, int gamma, float* surv, void* stream);

/*
 * W2 storage conversion.  The draft entry points take the r x V projection of
 * [P1] section 二 design 1 (Markov-head equation) stored column by column
 * (element (i, v) at W2[v * r + i]); this converts a row-by-row copy (element
 * (i, v) at w2_rv[i * V + v]) into that storage, once, when the weights are
 * loaded.  Off the drafting path.
 *   w2_rv     [r, V] bf16 device array (read).
 *   w2_store  [V, r] bf16 device array (written); must not overlap w2_rv.
 * Enqueued on `stream`; no host sync.  Errors: EINVAL for NULL pointers,
 * sizes <= 0 or overlapping arrays; EUNSUPPORTED for r above 4194240 or V
 * above 2^30 - 1; EDEVICE on a launch failure.
 */
dspark_status dspark_w2_store_from_rv(const uint16_t* w2_rv, int r, int V, uint16_t* w2_store,
                                     void* stream);

/* Bytes of workspace dspark_schedule needs (0 if invalid). */
size_t dspark_schedule_workspace(int R, int gamma);

/*
 * Hardware-aware prefix scheduler, [P1] section 二 design 2 (objective
 * Theta = tau * SPS(B), B = sum_r (1 + l_r), tau = sum_r (1 + sum_{j<=l_r} a_{r,j}),
 * global sort of candidates by survival) and section 三 challenge 2 (no early
 * stop: every budget is evaluated).  Candidates (r, j) carry id r*gamma + j-1
 * and key a_{r,j}; they are ordered by key descending, equal keys by id
 * ascending.  With q = rint(a * 2^40) and S_m the exact integer sum of the
 * first m ordered q's, Theta_m = double(R*2^40 + S_m) * 2^-40 * double(sps[R+m-1])
 * for m = 0..R*gamma; m* is the smallest m attaining the maximum, and l_r is
 * the number of request r's candidates among the first m* ordered ones.
 *
 *   surv      [R, gamma] fp32 survival probabilities (device data); values outside
 *             [0, 1] are clamped into it and NaN is taken as 0 (for the order,
 *             q and tau alike).
 *   sps       [B_max] fp32, sps[B-1] = SPS(B) >= 0, the engine's profiled steps/s.
 *   B_max     >= R * (1 + gamma).
 *   lengths   [R] int32 output l_r.
 *   order     optional [R * gamma] int32 output, the sorted candidate ids.
 *   info      optional dspark_schedule_info output (device memory).
 *   workspace >= dspark_schedule_workspace(R, gamma) bytes.
 * Errors: EINVAL for NULL required pointers, non-positive sizes or
 * B_max < R*(1+gamma); EUNSUPPORTED if R*gamma > DSPARK_MAX_CANDIDATES or
 * R*(1+gamma) >= 2^24; EWORKSPACE; EDEVICE.
 */
dspark_status dspark_schedule(const float* surv, const float* sps, int R, int gamma, int B_max,
                              int32_t* lengths, int32_t* order, dspark_schedule_info* info,
                              void* workspace, size_t ws_bytes, void* stream);

/* Admission rules of dspark_schedule_ex. */
typedef enum {
  DSPARK_SCHED_GLOBAL = 0,      /* global search over every budget (= dspark_schedule) */
  DSPARK_SCHED_EARLY_STOP = 1,  /* the greedy scan with its break */
  DSPARK_SCHED_CAPACITY = 2     /* a predicted batch capacity, top candidates */
} dspark_sched_mode;

/*
 * The scheduler with a choice of admission rule.  Candidates, their order,
 * q, S_m, Theta_m, l_r and the info fields are those of dspark_schedule.
 *   DSPARK_SCHED_GLOBAL: identical to dspark_schedule.
 *   DSPARK_SCHED_EARLY_STOP ([P1] section 二 design 2, greedy steps 3-5, the
 *     theoretical version that [P3] part 01 describes as non-anticipating):
 *     candidates are admitted in order while Theta keeps rising; m* is the
 *     smallest m with Theta_{m+1} <= Theta_m, or R*gamma if there is none.
 *   DSPARK_SCHED_CAPACITY ([P1] section 三 challenge 1, [P3] part 01: the
 *     asynchronous production form): `capacity` K is the predicted size of the
 *     next verification batch in tokens, anchors included; m* = clamp(K - R,
 *     0, R*gamma) (the dynamic top-K).  sps and B_max are not used (sps may be
 *     NULL); info->theta reports tau*.
 *   capacity  >= 0, used by DSPARK_SCHED_CAPACITY only.
 * Other arguments as for dspark_schedule; the workspace size is the same.
 * Errors: as dspark_schedule, plus EINVAL for an unknown mode or a negative
 * capacity (sps and B_max are checked only when the mode uses them).
 */
dspark_status dspark_schedule_ex(const float* surv, const float* sps, int R, int gamma, int B_max,
                                 int mode, int capacity, int32_t* lengths, int32_t* order,
                                 dspark_schedule_info* info, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Bytes of workspace dspark_draft_step needs (0 if invalid). */
size_t dspark_draft_step_workspace(int R, int gamma, int V, int r);

/*
 * Number of kernel launches one dspark_draft_step call makes for these sizes,
 * layout, mode and temperature, with W1 and w_conf + d 16-byte aligned (a
 * misaligned one can add the separate finishing launch).  Host-side planning
 * only (it reads the current device's properties); nothing is launched.
 * Errors: EINVAL for NULL count, bad sizes, unknown layout or mode, or a
 * non-positive sampling temperature.
 */
dspark_status dspark_draft_step_launches(int R, int gamma, int V, int r, int layout, int mode,
                                         float temperature, int* count);

/*
 * One whole drafting step of the head in one call: the gamma-step Markov-head
 * draft ([P1] section 二 design 1, as dspark_markov_draft), the confidence head
 * with STS and the prefix survivals ([P1] section 二 design 2, as
 * dspark_confidence), and the global-search schedule ([P1] section 二 design 2
 * and section 三 challenge 2, as dspark_schedule).  The results are those of
 * the three calls in sequence (up to the rounding order of the confidence
 * dot products).  It runs as a prologue that clears the draft's packed words
 * and computes the token-independent part w_h . h of every confidence logit,
 * then the gamma step kernels (whose first V group also computes
 * w_e . W1[x_{k-1}] from the rows it gathered), then the finishing work: the
 * sigmoid with STS, the survival products and the schedule.  That work needs
 * x_0 .. x_{gamma-2} only; where the last step's launch has a workgroup with
 * no step work (the rank-512 sampling kernel, whose V groups rarely fill the
 * launch), that workgroup does it beside the step, and the step workgroup
 * that finishes last unpacks the last tokens: gamma + 1 launches.  Otherwise
 * it is one launch after the last step (up to 8192 candidates; beyond that the
 * schedule's global path follows it): gamma + 2 or more.
 * dspark_draft_step_launches gives the count for given sizes.
 *   W1 ... uniforms   as for dspark_markov_draft (no bias output).
 *   h, w_conf, sts_temp, d   as for dspark_confidence; w_conf must be 16-byte
 *                            aligned and d a multiple of 4.
 *   sps, B_max               as for dspark_schedule.
 *   tokens, conf, surv       [R, gamma] outputs; lengths [R]; order [R*gamma]
 *                            and info optional, as for dspark_schedule.
 *   workspace  >= dspark_draft_step_workspace(R, gamma, V, r) bytes, 256-byte
 *              aligned; its contents on entry do not matter.
 *   events     optional per-step timing hooks of the gamma step kernels.
 * Errors: the union of the three calls' errors, plus EUNSUPPORTED for a
 * misaligned w_conf or d % 4 != 0 and EINVAL for a misaligned workspace.
 */
dspark_status dspark_draft_step(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const uint16_t* h, const float* w_conf, const float* sts_temp,
                                int d, const float* sps, int B_max, int32_t* tokens, float* conf,
                                float* surv, int32_t* lengths, int32_t* order,
                                dspark_schedule_info* info, void* workspace, size_t ws_bytes,
                                const dspark_step_events* events, void* stream);

/*
 * Verification side, [P1] section 三 challenge 3 (every verified token is one
 * flattened element; a marker tensor carries the within-sequence
 * dependencies) and [P3] Figure 1 (the target verifies anchor + kept prefix
 * in parallel).  Request r contributes 1 + l_r elements: its anchor, then its
 * first l_r drafts, at positions pos0[r] + j, each marked with r.
 *   anchors      [R] int32;  tokens [R, gamma] int32 drafts (row r, draft j at
 *                r*gamma + j - 1);  lengths [R] int32 l_r (values outside
 *                [0, gamma] are clamped into it).
 *   pos0         optional [R] int32 position of each anchor (0 if NULL).
 *   flat_tokens  [R*(1+gamma)] int32 output (the first B entries are written).
 *   flat_pos, flat_req  optional outputs of the same size: positions, request ids.
 *   cu_seqlens   [R+1] int32 output: segment starts, cu_seqlens[R] = B.
 * Errors: EINVAL for NULL required pointers or non-positive sizes;
 * EUNSUPPORTED if R*(1+gamma) exceeds 2^31 - 1; EDEVICE.
 */
dspark_status dspark_verify_pack(const int32_t* anchors, const int32_t* tokens,
                                 const int32_t* lengths, const int32_t* pos0, int R, int gamma,
                                 int32_t* flat_tokens, int32_t* flat_pos, int32_t* flat_req,
                                 int32_t* cu_seqlens, void* stream);

/*
 * Greedy verification of a flattened batch ([P3] Figure 1): t_e = argmax_v of
 * target_logits row e (the target's next token after element e; ties resolve to
 * the smallest id; rows must be free of NaN).  For request r with segment
 * start s = cu_seqlens[r] and l_r = cu_seqlens[r+1] - s - 1 drafts, drafts are
 * accepted while tokens[r, j] == t_{s+j}; accepted[r] = their number and
 * next_token[r] = t_{s + accepted[r]} (the correction of the first rejected
 * draft, or the bonus token when all are accepted).
 *   target_logits  [rows, V] fp32, row e for flattened element e (rows >= B;
 *                  rows from B on are not read).
 *   cu_seqlens     [R+1] as written by dspark_verify_pack.
 *   target_argmax  [R*(1+gamma)] int32 output (the first B entries are written).
 *   accepted, next_token  [R] int32 outputs.
 * Errors: EINVAL for NULL pointers or non-positive sizes; EUNSUPPORTED if
 * R*(1+gamma) exceeds 2^31 - 1; EDEVICE.
 */
dspark_status dspark_verify_greedy(const float* target_logits, const int32_t* cu_seqlens,
                                   const int32_t* tokens, int R, int gamma, int V,
                                   int32_t* target_argmax, int32_t* accepted,
                                   int32_t* next_token, void* stream);

/*
 * Acceptance probability of paired rows ([P1] section 二 design 2, the
 * confidence head's label 1 - TV(p_draft, p_target)):
 *   out[i] = sum_v min(softmax(draft_logits[i] / T)_v, softmax(target_logits[i] / T)_v).
 *   draft_logits, target_logits  [n, V] fp32 (each row needs a finite value;
 *                                -inf entries are allowed).
 *   temperature  T > 0 and finite.
 *   out          [n] fp32 output.
 * Errors: EINVAL for NULL pointers, non-positive sizes or a bad temperature;
 * EDEVICE.
 */
dspark_status dspark_accept_prob(const float* draft_logits, const float* target_logits, int n,
                                 int V, float temperature, float* out, void* stream);

/* Static description of a status code. */
const char* dspark_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* dspark_last_error(void);

/* Hash of the source files and compile flags this library was built from (32 hex
 * digits; "unknown" for a build outside the package's build script).  Loaders
 * compare it with the sources they ship to detect a stale library. */
const char* dspark_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
