// Markov-head step kernels: the variant table for kBiasOnly / kEpiNone (one
// translation unit per slice of the table, so the slices compile in parallel).
#include "markov_kernels.h"

namespace dspark {

StepVariant pick_bias_only(const MarkovPlan& p, bool bias) {
  return bias ? pick3<kBiasOnly, kEpiNone, true>(p) : pick3<kBiasOnly, kEpiNone, false>(p);
}

}  // namespace dspark
