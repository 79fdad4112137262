// Host side of the Markov-head draft: plan (kernel variant, grid, groups),
// the launches of a call, and the two small kernels around the steps.
//
// A call of dspark_markov_draft is gamma + 2 launches: one that clears the
// packed words, the gamma fused steps, and one that unpacks the last step's
// tokens.  The fused draft step (dspark_draft_step) replaces the clear with
// the confidence head's token-independent part and the unpack with the
// schedule: a prologue, the gamma steps (which also take the confidence
// head's embedding term), and a finishing launch.  (A last-arriving
// workgroup could do the unpack, but the device-scope release fence it needs
// costs more than the launch.)
#include <stdlib.h>

#include <mutex>

#include <hip/hip_ext.h>

#include "markov_types.h"
#include "packed_words.h"

namespace dspark {
namespace {

__global__ __launch_bounds__(256) void clear_words_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// tokens[m][k] from the packed results of the last step.
__global__ __launch_bounds__(256) void last_tokens_kernel(const unsigned long long* __restrict__ w,
                                                          int S, int R, int V, int gamma, int k,
                                                          int32_t* __restrict__ tokens) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m < R) tokens[(size_t)m * gamma + k] = read_token(w, m, S, V);
}

StepVariant pick_variant(const MarkovPlan& p, int mode, int epi, bool bias) {
  if (mode == kBiasOnly) return pick_bias_only(p, bias);
  if (mode == DSPARK_SAMPLE) return epi == kEpiCol ? pick_sample_col(p, bias) : pick_sample_row(p, bias);
  return epi == kEpiCol ? pick_greedy_col(p, bias) : pick_greedy_row(p, bias);
}

// Per-kernel launch attributes and occupancy, resolved once per variant and
// device (host threads may call concurrently).
struct VariantState {
  StepKernel fn;
  int device;
  int blocks_per_cu;
};
VariantState g_states[512];
int g_nstates = 0;
std::mutex g_states_mu;

int prepare_variant(const StepVariant& v) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(g_states_mu);
  for (int i = 0; i < g_nstates; ++i)
    if (g_states[i].fn == v.fn && g_states[i].device == dev) return g_states[i].blocks_per_cu;
  const void* f = reinterpret_cast<const void*>(v.fn);
  if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)v.lds) != hipSuccess)
    return -1;
  if (v.fn_fin && hipFuncSetAttribute(reinterpret_cast<const void*>(v.fn_fin),
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)v.lds) != hipSuccess)
    return -1;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, v.threads, v.lds) != hipSuccess || nb < 1)
    nb = 1;
  if (g_nstates < 512) g_states[g_nstates++] = {v.fn, dev, nb};
  return nb;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

// Everything the step launches of one call share.
struct DraftLaunch {
  StepVariant var;
  MarkovPlan p;
  dim3 grid;
  int cstep;
  int sub;             // packed words per request
  size_t words;        // R * sub
  size_t step_floats;  // tiled: floats of one step
  bool tiled;
  float inv_t;
  int kmode;
  int bpc;             // step workgroups that fit on one CU
};

dspark_status prepare_draft(int R, int gamma, int V, int r, int layout, int mode, float temperature,
                            bool have_base, bool bias, DraftLaunch& L) {
  // No base logits: greedy on the Markov bias alone.
  L.kmode = have_base ? mode : kBiasOnly;
  MarkovPlan p = plan_markov(R, gamma, V, r, L.kmode, true);
  L.tiled = layout == DSPARK_LAYOUT_TILED;
  const int epi = L.kmode == kBiasOnly ? kEpiNone : L.tiled ? kEpiCol : kEpiRow;
  L.var = pick_variant(p, L.kmode, epi, bias);
  p.n_rblocks = (R + L.var.rows - 1) / L.var.rows;   // the variant's requests per workgroup
  const int bpc = prepare_variant(L.var);
  if (bpc < 0) return fail(DSPARK_EDEVICE, "hipFuncSetAttribute failed for the Markov step kernel");
  L.bpc = bpc;

  // One wave of workgroups: as many as fit on the device at once, split between
  // the R blocks (each V group is walked by n_rblocks workgroups).  Groups hold
  // a multiple of the kernel's unroll factor of chunks.
  const int max_groups = p.n_chunks < kMaxGroups ? p.n_chunks : kMaxGroups;
  int target = env_int("DSPARK_MARKOV_WG", 0);
  if (target <= 0) target = device_cus() * (p.n_rblocks == 1 && R <= 64 && bpc > 2 ? 2 : bpc);
  if (target < 8) target = 8;
  int groups = (target + p.n_rblocks - 1) / p.n_rblocks;
  groups = (groups + 7) / 8 * 8;
  if (groups > max_groups) groups = max_groups;
  if (groups < 1) groups = 1;
  p.cpg = (p.n_chunks + groups - 1) / groups;
  p.cpg = (p.cpg + L.var.unroll - 1) / L.var.unroll * L.var.unroll;
  // Contiguous groups: group g owns chunks [g*cpg, (g+1)*cpg).  Strided groups:
  // group g owns chunks g, g + G, g + 2G, ... (all G groups in flight read one
  // contiguous window of W2 and of the logits at a time).  Strided groups
  // measured faster for the tiled layout at R >= 128 (sampling and long
  // blocks); DSPARK_MARKOV_STRIDED overrides.
  const int st_env = env_int("DSPARK_MARKOV_STRIDED", -1);
  const bool strided = st_env < 0 ? (L.tiled && R >= 128) : st_env != 0;
  p.n_vgroups = strided ? groups : (p.n_chunks + p.cpg - 1) / p.cpg;
  L.cstep = strided ? groups : 1;
  L.sub = p.n_vgroups > kSubWordsAboveGroups ? kMaxSubWords : 1;
  const int sub_env = env_int("DSPARK_MARKOV_SUBWORDS", 0);
  if (sub_env == 1 || sub_env == 2 || sub_env == 4 || sub_env == 8 || sub_env == 16) L.sub = sub_env;
  L.words = (size_t)R * L.sub;
  const int padded_groups = (p.n_vgroups + 7) / 8 * 8;
  L.grid = dim3(padded_groups * p.n_rblocks);
  L.inv_t = mode == DSPARK_SAMPLE ? 1.0f / temperature : 1.0f;
  // Column-tiled [gamma][C][32][R]: one step is C * 32 * R floats, and each
  // launch's range ends with its own step (rows past R are sent past it).
  L.step_floats = (size_t)p.n_chunks * kChunk * R;
  L.p = p;
  return DSPARK_OK;
}

// One fused step launch (position k).  `w_e` / `se` (optional) ask the step
// for the confidence head's embedding term; `dense` (optional) replaces the
// gathered W1 rows with dense [R, r] rows.
dspark_status launch_one_step(const DraftLaunch& L, int k, const uint16_t* W1, const uint16_t* W2,
                              const float* base, const int32_t* anchors, int R, int gamma, int V,
                              int r, const float* uniforms, int32_t* tokens, float* bias_out,
                              unsigned long long* packed, const float* w_e, float* se,
                              const uint16_t* dense, const dspark_step_events* events,
                              hipStream_t stream, const FinParams* fin = nullptr) {
  Addr ad;
  ad.row_stride = L.tiled ? 1 : (size_t)gamma * V;
  ad.cstride = L.tiled ? (size_t)kChunk * R : (size_t)kChunk;
  ad.vstride = L.tiled ? (size_t)R : 1;
  ad.total = (size_t)R * gamma * V;
  const StepIO io{anchors, k == 0 ? nullptr : packed + (size_t)(k - 1) * L.words,
                  packed + (size_t)k * L.words, tokens, gamma, k, L.sub, w_e, se, dense};
  ad.k_off = L.tiled ? (size_t)k * L.step_floats : (size_t)k * V;
  if (L.tiled) ad.total = ad.k_off + L.step_floats;
  // Timing hooks ride on the dispatch itself (start / stop timestamps of the
  // kernel's packet), so they add no marker packets between kernels.
  hipEvent_t ev_begin = nullptr, ev_end = nullptr;
  if (events && k < events->count) {
    if (events->begin) ev_begin = reinterpret_cast<hipEvent_t>(events->begin[k]);
    if (events->end) ev_end = reinterpret_cast<hipEvent_t>(events->end[k]);
  }
  if (fin)
    hipExtLaunchKernelGGL(L.var.fn_fin, L.grid, dim3(L.var.threads), (uint32_t)L.var.lds, stream,
                          ev_begin, ev_end, 0u, W1, W2, base, uniforms, io, R, V, r, L.inv_t,
                          L.p.n_rblocks, L.p.n_vgroups, L.p.cpg, L.cstep, L.p.n_chunks, ad,
                          bias_out, *fin);
  else
    hipExtLaunchKernelGGL(L.var.fn, L.grid, dim3(L.var.threads), (uint32_t)L.var.lds, stream,
                          ev_begin, ev_end, 0u, W1, W2, base, uniforms, io, R, V, r, L.inv_t,
                          L.p.n_rblocks, L.p.n_vgroups, L.p.cpg, L.cstep, L.p.n_chunks, ad,
                          bias_out);
  return check_launch("markov_step_kernel");
}

// The gamma fused step launches.
dspark_status launch_steps(const DraftLaunch& L, const uint16_t* W1, const uint16_t* W2,
                           const float* base, const int32_t* anchors, int R, int gamma, int V,
                           int r, const float* uniforms, int32_t* tokens, float* bias_out,
                           unsigned long long* packed, const float* w_e, float* se,
                           const uint16_t* dense, const dspark_step_events* events,
                           hipStream_t stream) {
  for (int k = 0; k < gamma; ++k) {
    const dspark_status st = launch_one_step(L, k, W1, W2, base, anchors, R, gamma, V, r, uniforms,
                                             tokens, bias_out, packed, w_e, se, dense, events,
                                             stream);
    if (st != DSPARK_OK) return st;
  }
  return DSPARK_OK;
}

}  // namespace

MarkovPlan plan_markov(int R, int gamma, int V, int r, int mode, bool for_launch) {
  (void)for_launch;
  MarkovPlan p{};
  p.rk = r <= 64 ? 64 : r <= 128 ? 128 : r <= 256 ? 256 : 512;
  const int waves_needed = (R + 31) / 32;
  int nw = waves_needed >= 8 ? 8 : waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1;
  // Choices measured on MI355X.  Rank 512 sampling: K-split wave pairs (a
  // plain wave would need the whole SIMD); rank 512 greedy: eight plain waves;
  // up to 64 requests: two-wave workgroups, at most two per CU (fewer,
  // longer groups).  DSPARK_MARKOV_KSPLIT / _NP / _NW / _WG / _STRIDED override the
  // choice for tuning (and DSPARK_MARKOV_SUBWORDS the words per request).
  if (p.rk == 512 && mode == DSPARK_SAMPLE && nw == 8) nw = 4;
  const int ks_env = env_int("DSPARK_MARKOV_KSPLIT", -1);
  p.ksplit = p.rk == 512 && (ks_env < 0 ? mode == DSPARK_SAMPLE : ks_env != 0);
  if (p.ksplit) nw = 2 * (waves_needed >= 4 ? 4 : waves_needed >= 2 ? 2 : 1);
  const int np_env = env_int("DSPARK_MARKOV_NP", 0);   // K-split wave pairs per workgroup
  if (p.ksplit && (np_env == 1 || np_env == 2 || np_env == 4)) nw = 2 * np_env;
  const int nw_env = env_int("DSPARK_MARKOV_NW", 0);
  if (!p.ksplit && (nw_env == 1 || nw_env == 2 || nw_env == 4 || nw_env == 8)) nw = nw_env;
  p.nw = nw;
  // Two tiles per wave halve the LDS reads per MFMA: the bias-only GEMM at
  // ranks 128-256 (DSPARK_MARKOV_TW=1 turns it off).  With bias output the
  // table has no such variant; the launch then falls back to one tile and
  // recomputes the R blocks from the variant's rows.
  const int tw_env = env_int("DSPARK_MARKOV_TW", 0);
  p.tw = (tw_env == 1 || tw_env == 2) ? tw_env : (mode == kBiasOnly ? 2 : 1);
  if (p.ksplit || (p.rk != 128 && p.rk != 256) || (nw != 4 && nw != 8) || mode != kBiasOnly)
    p.tw = 1;
  const int rows = p.ksplit ? nw / 2 * 32 : nw * 32 * p.tw;
  p.n_rblocks = (R + rows - 1) / rows;
  p.n_chunks = (V + kChunk - 1) / kChunk;
  // packed per-step results [gamma][R][S], sized for the largest S
  p.ws_bytes = (size_t)gamma * (size_t)R * kMaxSubWords * 8;
  return p;
}

dspark_status launch_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int layout, int mode, float temperature,
                                  const float* uniforms, int32_t* tokens, float* bias_out,
                                  void* workspace, const dspark_step_events* events,
                                  hipStream_t stream) {
  DraftLaunch L;
  dspark_status st = prepare_draft(R, gamma, V, r, layout, mode, temperature, base != nullptr,
                                   bias_out != nullptr, L);
  if (st != DSPARK_OK) return st;
  unsigned long long* packed = reinterpret_cast<unsigned long long*>(workspace);
  const size_t nclear = ((size_t)gamma * L.words + 1) / 2;   // 16-byte stores
  const size_t cblocks = (nclear + 255) / 256;
  hipLaunchKernelGGL(clear_words_kernel, dim3(cblocks < 1024 ? (unsigned)cblocks : 1024u),
                     dim3(256), 0, stream, reinterpret_cast<uint4*>(workspace), nclear);
  st = launch_steps(L, W1, W2, base, anchors, R, gamma, V, r, uniforms, tokens, bias_out, packed,
                    nullptr, nullptr, nullptr, events, stream);
  if (st != DSPARK_OK) return st;
  hipLaunchKernelGGL(last_tokens_kernel, dim3((R + 255) / 256), dim3(256), 0, stream,
                     packed + (size_t)(gamma - 1) * L.words, L.sub, R, V, gamma, gamma - 1,
                     tokens);
  return check_launch("last_tokens_kernel");
}

// The fused call's words: the packed per-step results, then the last step's
// count of finished workgroups (cleared with them).
size_t draft_step_words_bytes(int R, int gamma, int V, int r) {
  return plan_markov(R, gamma, V, r, DSPARK_GREEDY, false).ws_bytes + 16;
}

// The finishing work needs x_0 .. x_{gamma-2} only, so where the last step's
// launch has a workgroup without step work (a K-split variant with a
// finishing kernel, an empty V group in R block 0, every workgroup resident at
// once) it runs there, beside the step; else it is a launch of its own after
// the last step.  `aligned`: W1 and w_e 16-byte aligned.
static bool finish_in_last_step(const DraftLaunch& L, int R, int gamma, int r, bool aligned) {
  const int padded_groups = (int)L.grid.x / L.p.n_rblocks;
  return L.var.fn_fin && (long)R * gamma <= (long)kFinStepItems * L.var.threads &&
         padded_groups > L.p.n_vgroups && (long)L.grid.x <= (long)device_cus() * L.bpc &&
         r % 8 == 0 && aligned;
}

dspark_status draft_step_launch_count(int R, int gamma, int V, int r, int layout, int mode,
                                      float temperature, int* count) {
  DraftLaunch L;
  const dspark_status st = prepare_draft(R, gamma, V, r, layout, mode, temperature, true, false, L);
  if (st != DSPARK_OK) return st;
  const long N = (long)R * gamma;
  const int finish = finish_in_last_step(L, R, gamma, r, true) ? 0
                     : N <= 8192                              ? 1
                                                              : 1 + schedule_launch_count(R, gamma);
  *count = 1 + gamma + finish;
  return DSPARK_OK;
}

size_t draft_step_workspace_bytes(int R, int gamma, int V, int r) {
  const size_t words = draft_step_words_bytes(R, gamma, V, r);
  const size_t conf = (size_t)R * gamma * 3 * sizeof(float);   // sh, se (two halves)
  const size_t sched = schedule_workspace_bytes(R, gamma);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(words) + up(conf) + up(sched);
}

dspark_status launch_draft_step(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const uint16_t* h, const float* w_conf, const float* sts_temp,
                                int d, const float* sps, int32_t* tokens, float* conf,
                                float* surv, int32_t* lengths, int32_t* order,
                                dspark_schedule_info* info, void* workspace,
                                const dspark_step_events* events, hipStream_t stream) {
  DraftLaunch L;
  dspark_status st = prepare_draft(R, gamma, V, r, layout, mode, temperature, base != nullptr,
                                   false, L);
  if (st != DSPARK_OK) return st;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const size_t words_bytes = draft_step_words_bytes(R, gamma, V, r);
  unsigned long long* packed = reinterpret_cast<unsigned long long*>(ws);
  unsigned int* done = reinterpret_cast<unsigned int*>(packed + (size_t)gamma * L.words);
  float* sh = reinterpret_cast<float*>(ws + up(words_bytes));
  float* se = sh + (size_t)R * gamma;
  void* sched_ws = ws + up(words_bytes) + up((size_t)R * gamma * 3 * sizeof(float));
  // Prologue: clear the words the steps combine into (and the count after
  // them), and the hidden-state part of every confidence logit (it does not
  // depend on the draft).
  st = launch_conf_prologue(h, w_conf, R, gamma, d, sh, packed, (size_t)gamma * L.words + 2,
                            stream);
  if (st != DSPARK_OK) return st;
  const float* w_e = w_conf + d;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool in_step = finish_in_last_step(L, R, gamma, r, a16(W1) && a16(w_e));
  if (!in_step) {
    st = launch_steps(L, W1, W2, base, anchors, R, gamma, V, r, uniforms, tokens, nullptr, packed,
                      w_e, se, nullptr, events, stream);
    if (st != DSPARK_OK) return st;
    return launch_draft_finish(packed + (size_t)(gamma - 1) * L.words, L.sub, V, sh, se,
                               sts_temp, R, gamma, tokens, conf, surv, sps, lengths, order, info,
                               sched_ws, stream);
  }
  for (int k = 0; k + 1 < gamma; ++k) {
    st = launch_one_step(L, k, W1, W2, base, anchors, R, gamma, V, r, uniforms, tokens, nullptr,
                         packed, w_e, se, nullptr, events, stream);
    if (st != DSPARK_OK) return st;
  }
  FinParams fin{};
  fin.sh = sh;
  fin.sts = sts_temp;
  fin.sps = sps;
  fin.conf = conf;
  fin.surv = surv;
  fin.lengths = lengths;
  fin.order = order;
  fin.info = info;
  fin.done = done;
  return launch_one_step(L, gamma - 1, W1, W2, base, anchors, R, gamma, V, r, uniforms, tokens,
                         nullptr, packed, w_e, se, nullptr, events, stream, &fin);
}

dspark_status launch_rnn_draft(const uint16_t* W1, const uint16_t* W2, const uint16_t* U,
                               const float* b_rnn, const float* base, const uint16_t* h,
                               const int32_t* anchors, int R, int gamma, int V, int r, int d,
                               int layout, int mode, float temperature, const float* uniforms,
                               int32_t* tokens, float* state_out, void* workspace,
                               const dspark_step_events* events, hipStream_t stream) {
  DraftLaunch L;
  dspark_status st = prepare_draft(R, gamma, V, r, layout, mode, temperature, base != nullptr,
                                   false, L);
  if (st != DSPARK_OK) return st;
  const RnnBuffers B = rnn_buffers(workspace, R, gamma, V, r, d);
  st = launch_rnn_pre(h, U, b_rnn, R, gamma, r, d, B, (size_t)gamma * L.words, stream);
  if (st != DSPARK_OK) return st;
  for (int k = 0; k < gamma; ++k) {
    const unsigned long long* prev = k == 0 ? nullptr : B.words + (size_t)(k - 1) * L.words;
    // the last update may go to the caller's state output (no later step reads it)
    st = launch_rnn_state(W1, U, anchors, prev, L.sub, R, gamma, V, r, d, k, B,
                          k == gamma - 1 ? state_out : nullptr, stream);
    if (st != DSPARK_OK) return st;
    st = launch_one_step(L, k, W1, W2, base, anchors, R, gamma, V, r, uniforms, tokens, nullptr,
                         B.words, nullptr, nullptr, B.sb[(k + 1) & 1], events, stream);
    if (st != DSPARK_OK) return st;
  }
  hipLaunchKernelGGL(last_tokens_kernel, dim3((R + 255) / 256), dim3(256), 0, stream,
                     B.words + (size_t)(gamma - 1) * L.words, L.sub, R, V, gamma, gamma - 1,
                     tokens);
  return check_launch("last_tokens_kernel");
}

}  // namespace dspark
