// Internal declarations shared by the C-ABI layer and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

// Sets the thread-local error text and returns `st`.
dspark_status fail(dspark_status st, const char* fmt, ...);

// Maps a HIP error (e.g. from hipGetLastError after a launch) to a status.
dspark_status check_launch(const char* what);

// ---- Markov-head step (fused gather + MFMA bias GEMM + bias-add + select) ----

struct MarkovPlan {
  int rk;          // compiled rank bucket (64, 128, 256, 512)
  int nw;          // waves per workgroup (32 requests per wave, or per wave pair if ksplit)
  bool ksplit;     // rank-512 K-split pairs
  int tw;          // 32-request tiles per wave (plain kernel; 2 shares each LDS read)
  int n_rblocks;   // ceil(R / (32 * nw * tw))
  int n_chunks;    // ceil(V / 32): 32-column chunks of V
  int n_vgroups;   // groups of consecutive chunks, one per workgroup (per R block)
  int cpg;         // chunks per group
  size_t ws_bytes; // packed per-step results: gamma * R * 16 words of 8 bytes
};

// Host-visible argument checks of the draft (all but the workspace).
dspark_status check_markov_args(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const int32_t* tokens, const dspark_step_events* events);

// for_launch = false: only the static parts (buckets, workspace); no device queries.
MarkovPlan plan_markov(int R, int gamma, int V, int r, int mode, bool for_launch);

dspark_status launch_markov_draft(const uint16_t* W1, const uint16_t* W2, const float* base,
                                  const int32_t* anchors, int R, int gamma, int V, int r,
                                  int layout, int mode, float temperature,
                                  const float* uniforms, int32_t* tokens, float* bias_out,
                                  void* workspace, const dspark_step_events* events,
                                  hipStream_t stream);

// ---- fused draft step: draft + confidence + survival + schedule ----
size_t draft_step_workspace_bytes(int R, int gamma, int V, int r);
dspark_status launch_draft_step(const uint16_t* W1, const uint16_t* W2, const float* base,
                                const int32_t* anchors, int R, int gamma, int V, int r,
                                int layout, int mode, float temperature, const float* uniforms,
                                const uint16_t* h, const float* w_conf, const float* sts_temp,
                                int d, const float* sps, int32_t* tokens, float* conf,
                                float* surv, int32_t* lengths, int32_t* order,
                                dspark_schedule_info* info, void* workspace,
                                const dspark_step_events* events, hipStream_t stream);
// Kernel launches of one launch_draft_step (W1 and w_e 16-byte aligned), and
// of one launch_schedule.
dspark_status draft_step_launch_count(int R, int gamma, int V, int r, int layout, int mode,
                                      float temperature, int* count);
int schedule_launch_count(int R, int gamma);
// Clears n_words packed words and writes sh[m * gamma + k] = w_h . h[m, k, :].
dspark_status launch_conf_prologue(const uint16_t* h, const float* w_h, int R, int gamma, int d,
                                   float* sh, unsigned long long* words, size_t n_words,
                                   hipStream_t stream);
// Last tokens from the packed words, c = sigmoid((sh + se0 + se1) / T_k),
// survival, then the global-search schedule.
dspark_status launch_draft_finish(const unsigned long long* words_last, int S, int V,
                                  const float* sh, const float* se, const float* sts_temp, int R,
                                  int gamma, int32_t* tokens, float* conf, float* surv,
                                  const float* sps, int32_t* lengths, int32_t* order,
                                  dspark_schedule_info* info, void* sched_ws, hipStream_t stream);

// ---- RNN head ----
// Workspace of the RNN-head draft: packed words, the token-independent
// pre-activations as `splits` partial sums P [splits][R * gamma][2r] fp32, and a
// ping-pong pair of states in fp32 and in bf16 ([2][R][r] each).
struct RnnBuffers {
  unsigned long long* words;
  size_t words_bytes;
  int splits;
  float* P;
  float* s[2];
  uint16_t* sb[2];
};
int rnn_pre_splits(int R, int gamma, int r, int d);
size_t rnn_workspace_bytes(int R, int gamma, int V, int r, int d);
RnnBuffers rnn_buffers(void* workspace, int R, int gamma, int V, int r, int d);
dspark_status launch_rnn_pre(const uint16_t* h, const uint16_t* U, const float* b, int R,
                             int gamma, int r, int d, const RnnBuffers& B, size_t n_words,
                             hipStream_t stream);
dspark_status launch_rnn_state(const uint16_t* W1, const uint16_t* U, const int32_t* anchors,
                               const unsigned long long* prev, int sub, int R, int gamma, int V,
                               int r, int d, int k, const RnnBuffers& B, float* s_out,
                               hipStream_t stream);
dspark_status launch_rnn_draft(const uint16_t* W1, const uint16_t* W2, const uint16_t* U,
                               const float* b_rnn, const float* base, const uint16_t* h,
                               const int32_t* anchors, int R, int gamma, int V, int r, int d,
                               int layout, int mode, float temperature, const float* uniforms,
                               int32_t* tokens, float* state_out, void* workspace,
                               const dspark_step_events* events, hipStream_t stream);

// ---- confidence head + survival ----
dspark_status launch_confidence(const uint16_t* h, const uint16_t* W1, const int32_t* anchors,
                                const int32_t* tokens, const float* w_conf, const float* sts_temp,
                                int R, int gamma, int d, int V, int r, float* conf, float* surv,
                                hipStream_t stream);
dspark_status launch_survival(const float* conf, int R, int gamma, float* surv, hipStream_t stream);
dspark_status launch_w2_store_from_rv(const uint16_t* w2_rv, uint16_t* w2_store, int r, int V,
                                      hipStream_t stream);

// ---- verification side ----
dspark_status launch_verify_pack(const int32_t* anchors, const int32_t* tokens,
                                 const int32_t* lengths, const int32_t* pos0, int R, int gamma,
                                 int32_t* flat_tokens, int32_t* flat_pos, int32_t* flat_req,
                                 int32_t* cu_seqlens, hipStream_t stream);
dspark_status launch_verify_greedy(const float* target_logits, const int32_t* cu_seqlens,
                                   const int32_t* tokens, int R, int gamma, int V,
                                   int32_t* target_argmax, int32_t* accepted,
                                   int32_t* next_token, hipStream_t stream);
dspark_status launch_accept_prob(const float* draft_logits, const float* target_logits, int n,
                                 int V, float temperature, float* out, hipStream_t stream);

// ---- prefix scheduler ----
dspark_status check_schedule_sizes(int R, int gamma, int B_max, bool uses_sps, const char* who);
size_t schedule_workspace_bytes(int R, int gamma);
// mode: 0 global search, 1 early stop, 2 capacity (m_cap = clamp(K - R, 0, R * gamma)).
dspark_status launch_schedule(const float* surv, const float* sps, int R, int gamma, int mode,
                              int m_cap, int32_t* lengths, int32_t* order,
                              dspark_schedule_info* info, void* workspace, hipStream_t stream);

}  // namespace dspark
