// Markov-head step kernels: the variant table for DSPARK_SAMPLE / kEpiRow (one
// translation unit per slice of the table, so the slices compile in parallel).
#include "markov_kernels.h"

namespace dspark {

StepVariant pick_sample_row(const MarkovPlan& p, bool bias) {
  return bias ? pick3<DSPARK_SAMPLE, kEpiRow, true>(p) : pick3<DSPARK_SAMPLE, kEpiRow, false>(p);
}

}  // namespace dspark
