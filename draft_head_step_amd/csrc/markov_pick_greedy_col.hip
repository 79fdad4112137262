// Markov-head step kernels: the variant table for DSPARK_GREEDY / kEpiCol (one
// translation unit per slice of the table, so the slices compile in parallel).
#include "markov_kernels.h"

namespace dspark {

StepVariant pick_greedy_col(const MarkovPlan& p, bool bias) {
  return bias ? pick3<DSPARK_GREEDY, kEpiCol, true>(p) : pick3<DSPARK_GREEDY, kEpiCol, false>(p);
}

}  // namespace dspark
