// Markov-head step kernels: the variant table for DSPARK_SAMPLE / kEpiCol (one
// translation unit per slice of the table, so the slices compile in parallel).
#include "markov_kernels.h"

namespace dspark {

StepVariant pick_sample_col(const MarkovPlan& p, bool bias) {
  return bias ? pick3<DSPARK_SAMPLE, kEpiCol, true>(p) : pick3<DSPARK_SAMPLE, kEpiCol, false>(p);
}

}  // namespace dspark
