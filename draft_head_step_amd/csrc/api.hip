// C ABI entry points: host-side argument validation, then kernel launches.
// Every check below runs before anything is enqueued; a failing check returns
// a status and leaves the stream untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "dspark_internal.h"

namespace dspark {
namespace {
thread_local char g_last_error[512] = "";
}  // namespace

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dspark_status fail(dspark_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

dspark_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSPARK_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return DSPARK_OK;
}

// Host-visible argument checks of the Markov-head draft (everything except the
// workspace), shared by the entry points that launch it.
dspark_status check_markov_args(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const int32_t* tokens, const dspark_step_events* events) {
  if (!W1 || !W2 || !anchors || !tokens)
    return fail(DSPARK_EINVAL, "markov_draft: NULL required pointer");
  if (!base && mode != DSPARK_GREEDY)
    return fail(DSPARK_EINVAL, "markov_draft: base may be NULL only in GREEDY mode");
  if (R <= 0 || gamma <= 0 || r <= 0 || V < 2)
    return fail(DSPARK_EINVAL, "markov_draft: need R, gamma, r > 0 and V >= 2 (got %d %d %d %d)",
                R, gamma, r, V);
  if (layout != DSPARK_LAYOUT_RGV && layout != DSPARK_LAYOUT_TILED)
    return fail(DSPARK_EINVAL, "markov_draft: unknown layout %d", layout);
  if (mode != DSPARK_GREEDY && mode != DSPARK_SAMPLE)
    return fail(DSPARK_EINVAL, "markov_draft: unknown mode %d", mode);
  if (mode == DSPARK_SAMPLE) {
    if (!uniforms) return fail(DSPARK_EINVAL, "markov_draft: SAMPLE needs uniforms");
    if (!(temperature > 0.0f) || !isfinite(temperature))
      return fail(DSPARK_EINVAL, "markov_draft: SAMPLE needs a positive finite temperature");
  } else if (uniforms) {
    return fail(DSPARK_EINVAL, "markov_draft: uniforms given in GREEDY mode");
  }
  if (!aligned16(W1) || !aligned16(W2))
    return fail(DSPARK_EINVAL, "markov_draft: W1 and W2 must be 16-byte aligned");
  if (r > DSPARK_MAX_RANK || r % 16 != 0)
    return fail(DSPARK_EUNSUPPORTED, "markov_draft: r must be a multiple of 16 and <= %d (got %d)",
                DSPARK_MAX_RANK, r);
  {
    // The kernels address each step's slice of one request block with 32-bit
    // byte offsets (buffer loads).
    const uint64_t C = ((uint64_t)V + 31) / 32;
    if (C * 32 * (uint64_t)r > (1ull << 30))
      return fail(DSPARK_EUNSUPPORTED, "markov_draft: ceil(V/32)*32*r above 2^30");
    if (layout == DSPARK_LAYOUT_RGV && (uint64_t)gamma * (uint64_t)V >= (1ull << 22))
      return fail(DSPARK_EUNSUPPORTED, "markov_draft: gamma*V must be below 2^22 in the RGV layout");
    // Tiled: one step (C * 32 * R floats) stays below 2^31 bytes, so an offset
    // pushed out of range by 2^31 is never back in range.
    if (layout == DSPARK_LAYOUT_TILED && C * (uint64_t)R >= (1ull << 24))
      return fail(DSPARK_EUNSUPPORTED, "markov_draft: ceil(V/32)*R must be below 2^24 in the tiled layout");
  }
  if (events && (events->count < gamma))
    return fail(DSPARK_EINVAL, "markov_draft: events->count < gamma");
  return DSPARK_OK;
}

// Size checks of the scheduler: B_max covers every budget (when an SPS table
// is used), R * gamma within the candidate limit, and R * (1 + gamma) < 2^24 so
// the fixed-point tau (at most R (1 + gamma) 2^40 with survivals in [0, 1])
// stays below 2^64.
dspark_status check_schedule_sizes(int R, int gamma, int B_max, bool uses_sps, const char* who) {
  if (R <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "%s: sizes must be positive", who);
  if (uses_sps && (long long)B_max < (long long)R * (1LL + gamma))
    return fail(DSPARK_EINVAL, "%s: B_max %d < R * (1 + gamma)", who, B_max);
  if ((long long)R * gamma > DSPARK_MAX_CANDIDATES)
    return fail(DSPARK_EUNSUPPORTED, "%s: R * gamma above %d", who, DSPARK_MAX_CANDIDATES);
  if ((long long)R * (1LL + gamma) >= (1LL << 24))
    return fail(DSPARK_EUNSUPPORTED, "%s: R * (1 + gamma) must be below 2^24", who);
  return DSPARK_OK;
}

}  // namespace dspark

using dspark::aligned16;
using dspark::fail;

extern "C" {

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_EINVAL: return "invalid argument";
    case DSPARK_EWORKSPACE: return "workspace too small";
    case DSPARK_EUNSUPPORTED: return "unsupported size";
    case DSPARK_EDEVICE: return "device error";
    default: return "unknown status";
  }
}

const char* dspark_last_error(void) { return dspark::g_last_error; }

#ifndef DSPARK_SOURCE_HASH
#define DSPARK_SOURCE_HASH "unknown"
#endif
const char* dspark_source_hash(void) { return DSPARK_SOURCE_HASH; }

size_t dspark_markov_draft_workspace(int R, int gamma, int V, int r) {
  if (R <= 0 || gamma <= 0 || V < 2 || r <= 0) return 0;
  return dspark::plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes;
}

dspark_status dspark_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int layout, int mode, float temperature, const float* uniforms,
                                  int32_t* tokens, float* bias_out, void* workspace,
                                  size_t ws_bytes, const dspark_step_events* events,
                                  void* stream) {
  dspark::g_last_error[0] = 0;
  const dspark_status st = dspark::check_markov_args(W1, W2, base, anchors, R, gamma, V, r, layout,
                                                     mode, temperature, uniforms, tokens, events);
  if (st != DSPARK_OK) return st;
  const size_t need = dspark_markov_draft_workspace(R, gamma, V, r);
  if (!workspace || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "markov_draft: workspace needs %zu bytes (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  if (!aligned16(workspace))
    return fail(DSPARK_EINVAL, "markov_draft: workspace must be 16-byte aligned");
  return dspark::launch_markov_draft(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                     temperature, uniforms, tokens, bias_out, workspace, events,
                                     reinterpret_cast<hipStream_t>(stream));
}

size_t dspark_draft_step_workspace(int R, int gamma, int V, int r) {
  if (R <= 0 || gamma <= 0 || V < 2 || r <= 0) return 0;
  if ((long long)R * gamma > DSPARK_MAX_CANDIDATES) return 0;
  if ((long long)R * (1LL + gamma) >= (1LL << 24)) return 0;
  return dspark::draft_step_workspace_bytes(R, gamma, V, r);
}

dspark_status dspark_draft_step_launches(int R, int gamma, int V, int r, int layout, int mode,
                                        float temperature, int* count) {
  dspark::g_last_error[0] = 0;
  if (!count) return fail(DSPARK_EINVAL, "draft_step_launches: NULL count");
  if (R <= 0 || gamma <= 0 || V < 2 || r <= 0 || r > DSPARK_MAX_RANK)
    return fail(DSPARK_EINVAL, "draft_step_launches: bad sizes R=%d gamma=%d V=%d r=%d", R, gamma,
                V, r);
  if (layout != DSPARK_LAYOUT_RGV && layout != DSPARK_LAYOUT_TILED)
    return fail(DSPARK_EINVAL, "draft_step_launches: unknown layout %d", layout);
  if (mode != DSPARK_GREEDY && mode != DSPARK_SAMPLE)
    return fail(DSPARK_EINVAL, "draft_step_launches: unknown mode %d", mode);
  if (mode == DSPARK_SAMPLE && !(temperature > 0.0f))
    return fail(DSPARK_EINVAL, "draft_step_launches: temperature must be positive");
  return dspark::draft_step_launch_count(R, gamma, V, r, layout, mode, temperature, count);
}

dspark_status dspark_draft_step(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const uint16_t* h, const float* w_conf, const float* sts_temp,
                                int d, const float* sps, int B_max, int32_t* tokens, float* conf,
                                float* surv, int32_t* lengths, int32_t* order,
                                dspark_schedule_info* info, void* workspace, size_t ws_bytes,
                                const dspark_step_events* events, void* stream) {
  dspark::g_last_error[0] = 0;
  dspark_status st = dspark::check_markov_args(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                               temperature, uniforms, tokens, events);
  if (st != DSPARK_OK) return st;
  if (!h || !w_conf || !sps || !conf || !surv || !lengths)
    return fail(DSPARK_EINVAL, "draft_step: NULL required pointer");
  if (d <= 0) return fail(DSPARK_EINVAL, "draft_step: d must be positive (got %d)", d);
  if (!aligned16(w_conf) || d % 4 != 0)
    return fail(DSPARK_EUNSUPPORTED, "draft_step: w_conf must be 16-byte aligned and d a multiple of 4");
  st = dspark::check_schedule_sizes(R, gamma, B_max, true, "draft_step");
  if (st != DSPARK_OK) return st;
  const size_t need = dspark_draft_step_workspace(R, gamma, V, r);
  if (!workspace || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "draft_step: workspace needs %zu bytes (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DSPARK_EINVAL, "draft_step: workspace must be 256-byte aligned");
  return dspark::launch_draft_step(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                   temperature, uniforms, h, w_conf, sts_temp, d, sps, tokens,
                                   conf, surv, lengths, order, info, workspace, events,
                                   reinterpret_cast<hipStream_t>(stream));
}

size_t dspark_rnn_draft_workspace(int R, int gamma, int V, int r, int d) {
  if (R <= 0 || gamma <= 0 || V < 2 || r <= 0 || d <= 0) return 0;
  return dspark::rnn_workspace_bytes(R, gamma, V, r, d);
}

dspark_status dspark_rnn_draft(const uint16_t* W1, const uint16_t* W2, const uint16_t* U,
                               const float* b_rnn, const float* base, const uint16_t* h,
                               const int32_t* anchors, int R, int gamma, int V, int r, int d,
                               int layout, int mode, float temperature, const float* uniforms,
                               int32_t* tokens, float* state_out, void* workspace, size_t ws_bytes,
                               const dspark_step_events* events, void* stream) {
  dspark::g_last_error[0] = 0;
  dspark_status st = dspark::check_markov_args(W1, W2, base, anchors, R, gamma, V, r, layout, mode,
                                               temperature, uniforms, tokens, events);
  if (st != DSPARK_OK) return st;
  if (!U || !b_rnn || !h) return fail(DSPARK_EINVAL, "rnn_draft: NULL required pointer");
  if (d <= 0) return fail(DSPARK_EINVAL, "rnn_draft: d must be positive (got %d)", d);
  if (d % 8 != 0 || !aligned16(U) || !aligned16(h))
    return fail(DSPARK_EUNSUPPORTED, "rnn_draft: d must be a multiple of 8 and U, h 16-byte aligned");
  if ((long long)R * gamma * 2LL * r >= (1LL << 31))
    return fail(DSPARK_EUNSUPPORTED, "rnn_draft: R * gamma * 2r must be below 2^31");
  if (2 * (int64_t)r + d > (1 << 22))
    return fail(DSPARK_EUNSUPPORTED, "rnn_draft: 2r + d must be at most 2^22 (got %lld)",
                (long long)(2 * (int64_t)r + d));
  const size_t need = dspark_rnn_draft_workspace(R, gamma, V, r, d);
  if (!workspace || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "rnn_draft: workspace needs %zu bytes (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(DSPARK_EINVAL, "rnn_draft: workspace must be 256-byte aligned");
  return dspark::launch_rnn_draft(W1, W2, U, b_rnn, base, h, anchors, R, gamma, V, r, d, layout,
                                  mode, temperature, uniforms, tokens, state_out, workspace, events,
                                  reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_confidence(const uint16_t* h, const uint16_t* W1, const int32_t* anchors,
                                const int32_t* tokens, const float* w_conf,
                                const float* sts_temp, int R, int gamma, int d, int V, int r,
                                float* conf, float* surv, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!h || !W1 || !anchors || !tokens || !w_conf || !conf)
    return fail(DSPARK_EINVAL, "confidence: NULL required pointer");
  if (R <= 0 || gamma <= 0 || d <= 0 || V <= 0 || r <= 0)
    return fail(DSPARK_EINVAL, "confidence: sizes must be positive");
  return dspark::launch_confidence(h, W1, anchors, tokens, w_conf, sts_temp, R, gamma, d, V, r,
                                   conf, surv, reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_survival(const float* conf, int R, int gamma, float* surv, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!conf || !surv) return fail(DSPARK_EINVAL, "survival: NULL required pointer");
  if (R <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "survival: sizes must be positive");
  if (conf == surv) return fail(DSPARK_EINVAL, "survival: conf and surv may not alias");
  return dspark::launch_survival(conf, R, gamma, surv, reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_w2_store_from_rv(const uint16_t* w2_rv, int r, int V, uint16_t* w2_store,
                                     void* stream) {
  dspark::g_last_error[0] = 0;
  if (!w2_rv || !w2_store) return fail(DSPARK_EINVAL, "w2_store_from_rv: NULL required pointer");
  if (r <= 0 || V <= 0) return fail(DSPARK_EINVAL, "w2_store_from_rv: sizes must be positive");
  // grid: ceil(V/64) x ceil(r/64) tiles of 256 threads (y at most 65535; the x
  // dimension's work-items below 2^32)
  if (r > 64 * 65535 || V >= (1 << 30))
    return fail(DSPARK_EUNSUPPORTED, "w2_store_from_rv: r above 4194240 or V above 2^30 - 1");
  const char* a = reinterpret_cast<const char*>(w2_rv);
  const char* b = reinterpret_cast<const char*>(w2_store);
  const size_t n = (size_t)r * (size_t)V * 2;
  if (a < b + n && b < a + n)
    return fail(DSPARK_EINVAL, "w2_store_from_rv: source and destination may not overlap");
  return dspark::launch_w2_store_from_rv(w2_rv, w2_store, r, V,
                                         reinterpret_cast<hipStream_t>(stream));
}

size_t dspark_schedule_workspace(int R, int gamma) {
  if (R <= 0 || gamma <= 0) return 0;
  if ((long long)R * gamma > DSPARK_MAX_CANDIDATES) return 0;
  if ((long long)R * (1LL + gamma) >= (1LL << 24)) return 0;
  return dspark::schedule_workspace_bytes(R, gamma);
}

dspark_status dspark_schedule(const float* surv, const float* sps, int R, int gamma, int B_max,
                              int32_t* lengths, int32_t* order, dspark_schedule_info* info,
                              void* workspace, size_t ws_bytes, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!surv || !sps || !lengths) return fail(DSPARK_EINVAL, "schedule: NULL required pointer");
  const dspark_status sz = dspark::check_schedule_sizes(R, gamma, B_max, true, "schedule");
  if (sz != DSPARK_OK) return sz;
  const size_t need = dspark_schedule_workspace(R, gamma);
  if (!workspace || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "schedule: workspace needs %zu bytes (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  return dspark::launch_schedule(surv, sps, R, gamma, 0, 0, lengths, order, info, workspace,
                                 reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_schedule_ex(const float* surv, const float* sps, int R, int gamma, int B_max,
                                 int mode, int capacity, int32_t* lengths, int32_t* order,
                                 dspark_schedule_info* info, void* workspace, size_t ws_bytes,
                                 void* stream) {
  dspark::g_last_error[0] = 0;
  if (mode != DSPARK_SCHED_GLOBAL && mode != DSPARK_SCHED_EARLY_STOP &&
      mode != DSPARK_SCHED_CAPACITY)
    return fail(DSPARK_EINVAL, "schedule_ex: unknown mode %d", mode);
  const bool uses_sps = mode != DSPARK_SCHED_CAPACITY;
  if (!surv || !lengths || (uses_sps && !sps))
    return fail(DSPARK_EINVAL, "schedule_ex: NULL required pointer");
  if (R <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "schedule_ex: sizes must be positive");
  if (mode == DSPARK_SCHED_CAPACITY && capacity < 0)
    return fail(DSPARK_EINVAL, "schedule_ex: negative capacity %d", capacity);
  const dspark_status sz = dspark::check_schedule_sizes(R, gamma, B_max, uses_sps, "schedule_ex");
  if (sz != DSPARK_OK) return sz;
  const size_t need = dspark_schedule_workspace(R, gamma);
  if (!workspace || ws_bytes < need)
    return fail(DSPARK_EWORKSPACE, "schedule_ex: workspace needs %zu bytes (got %zu)", need,
                workspace ? ws_bytes : (size_t)0);
  const long long n = (long long)R * gamma;
  long long m_cap = (long long)capacity - R;
  m_cap = m_cap < 0 ? 0 : m_cap > n ? n : m_cap;
  return dspark::launch_schedule(surv, uses_sps ? sps : nullptr, R, gamma, mode, (int)m_cap,
                                 lengths, order, info, workspace,
                                 reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_verify_pack(const int32_t* anchors, const int32_t* tokens,
                                 const int32_t* lengths, const int32_t* pos0, int R, int gamma,
                                 int32_t* flat_tokens, int32_t* flat_pos, int32_t* flat_req,
                                 int32_t* cu_seqlens, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!anchors || !tokens || !lengths || !flat_tokens || !cu_seqlens)
    return fail(DSPARK_EINVAL, "verify_pack: NULL required pointer");
  if (R <= 0 || gamma <= 0) return fail(DSPARK_EINVAL, "verify_pack: sizes must be positive");
  if ((long long)R * (1LL + gamma) > 0x7fffffffLL)
    return fail(DSPARK_EUNSUPPORTED, "verify_pack: R * (1 + gamma) above 2^31 - 1");
  return dspark::launch_verify_pack(anchors, tokens, lengths, pos0, R, gamma, flat_tokens,
                                    flat_pos, flat_req, cu_seqlens,
                                    reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_verify_greedy(const float* target_logits, const int32_t* cu_seqlens,
                                   const int32_t* tokens, int R, int gamma, int V,
                                   int32_t* target_argmax, int32_t* accepted,
                                   int32_t* next_token, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!target_logits || !cu_seqlens || !tokens || !target_argmax || !accepted || !next_token)
    return fail(DSPARK_EINVAL, "verify_greedy: NULL required pointer");
  if (R <= 0 || gamma <= 0 || V < 1)
    return fail(DSPARK_EINVAL, "verify_greedy: sizes must be positive");
  if ((long long)R * (1LL + gamma) > 0x7fffffffLL)
    return fail(DSPARK_EUNSUPPORTED, "verify_greedy: R * (1 + gamma) above 2^31 - 1");
  return dspark::launch_verify_greedy(target_logits, cu_seqlens, tokens, R, gamma, V,
                                      target_argmax, accepted, next_token,
                                      reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_accept_prob(const float* draft_logits, const float* target_logits, int n,
                                 int V, float temperature, float* out, void* stream) {
  dspark::g_last_error[0] = 0;
  if (!draft_logits || !target_logits || !out)
    return fail(DSPARK_EINVAL, "accept_prob: NULL required pointer");
  if (n <= 0 || V < 1) return fail(DSPARK_EINVAL, "accept_prob: sizes must be positive");
  if (!(temperature > 0.0f) || !isfinite(temperature))
    return fail(DSPARK_EINVAL, "accept_prob: temperature must be positive and finite");
  return dspark::launch_accept_prob(draft_logits, target_logits, n, V, temperature, out,
                                    reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
