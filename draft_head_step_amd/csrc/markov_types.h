// Types shared by the Markov-head step kernels (markov_kernels.h, instantiated
// in the markov_pick_*.hip units) and their host launcher (markov_step.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dspark_internal.h"

namespace dspark {

constexpr int kChunk = 32;         // vocabulary rows of W2 per MFMA tile
constexpr int kMaxGroups = 1024;   // upper bound on V groups (sizes the workspace)
// Internal mode: greedy on the Markov bias alone (no base logits are read).
constexpr int kBiasOnly = 2;

// How a step kernel reads the logits and uniforms of a chunk, which also
// fixes which MFMA operand the requests are:
//   kEpiNone  no logits stream (bias only); requests on the lanes;
//   kEpiCol   column-tiled logits ([gamma][C][32][R]); requests on the lanes, so
//             one four-byte load of a vocabulary entry for a 32-request tile
//             reads a whole 128-byte line;
//   kEpiRow   row-major logits ([R][gamma][V]); vocabulary entries on the
//             lanes (the bias tile is computed untransposed), so one four-byte
//             load of a request's 32 entries in a half-wave reads a whole line.
constexpr int kEpiNone = 0;
constexpr int kEpiCol = 1;
constexpr int kEpiRow = 2;

// Items per thread of the finishing schedule inside the fused step's last
// step (see StepIO): it covers R gamma <= 4 x the K-split workgroup's threads.
constexpr int kFinStepItems = 4;

// Where a step kernel takes its input tokens and leaves its results.
struct StepIO {
  const int32_t* anchors;              // step 0: x_0
  const unsigned long long* prev;      // steps > 0: packed results of step k-1 [R][sub]
  unsigned long long* best;            // packed results of step k, cleared before step 0
  int32_t* tokens;                     // [R][gamma]
  int gamma;
  int k;
  int sub;                             // words per request (power of two)
  // Embedding part of the confidence logit (fused draft step, optional): the
  // first V group of each R block writes w_e . W1[x_{k-1}] of its requests to
  // se[(m * gamma + k) * 2 + h], h = 0, 1 the two K halves of the K-split
  // kernel (the plain kernel writes the whole dot to h = 0 and 0 to h = 1);
  // NaN where x_{k-1} is not a valid id.
  const float* w_e;                    // [r] or NULL
  float* se;                           // [R][gamma][2] or NULL
  // Rows of the bias GEMM from a dense [R, r] bf16 array (row m for request m)
  // instead of the gathered W1[x_{k-1}] (NULL: gather).
  const uint16_t* dense;
};

// The fused draft step's last step (a variant's fn_fin): the finishing work
// (confidences, STS, survivals and the schedule, which need x_0 .. x_{gamma-2}
// only) runs on the workgroup of R block 0's first empty V group, beside the
// step workgroups, and the step workgroup that finishes last writes x_{gamma-1}
// to tokens.  A kernel argument of that launch only.
struct FinParams {
  const float* sh;                     // w_h . h [R][gamma]
  const float* sts;                    // [gamma] or NULL
  const float* sps;                    // SPS table
  float* conf;                         // [R][gamma]
  float* surv;                         // [R][gamma]
  int32_t* lengths;                    // [R]
  int32_t* order;                      // [R * gamma] or NULL
  dspark_schedule_info* info;          // or NULL
  unsigned int* done;                  // step workgroups finished, 0 before the step
};

// Element (m, k, v) of base / uniforms / bias_out is at float offset
// k_off + m * row_stride + (v / 32) * cstride + (v % 32) * vstride in either
// layout; the kernels' resources cover [block start, total).  Byte offsets
// inside one R block of one step fit in 32 bits (checked on the host).
struct Addr {
  size_t k_off, row_stride, cstride, vstride, total;
};

using StepKernel = void (*)(const uint16_t*, const uint16_t*, const float*, const float*,
                            StepIO, int, int, int, float, int, int, int, int, int, Addr, float*);
using StepFinKernel = void (*)(const uint16_t*, const uint16_t*, const float*, const float*,
                               StepIO, int, int, int, float, int, int, int, int, int, Addr,
                               float*, FinParams);

struct StepVariant {
  StepKernel fn;
  int threads;
  size_t lds;
  int rows;     // requests per workgroup
  int unroll;   // chunks per group must be a multiple of this
  StepFinKernel fn_fin;   // the fused step's last step with its finishing work, or NULL
};

// Kernel tables, one translation unit each (they compile in parallel).
StepVariant pick_greedy_row(const MarkovPlan& p, bool bias);
StepVariant pick_greedy_col(const MarkovPlan& p, bool bias);
StepVariant pick_sample_row(const MarkovPlan& p, bool bias);
StepVariant pick_sample_col(const MarkovPlan& p, bool bias);
StepVariant pick_bias_only(const MarkovPlan& p, bool bias);

}  // namespace dspark
