// Markov-head step kernels: the variant table for DSPARK_GREEDY / kEpiRow (one
// translation unit per slice of the table, so the slices compile in parallel).
#include "markov_kernels.h"

namespace dspark {

StepVariant pick_greedy_row(const MarkovPlan& p, bool bias) {
  return bias ? pick3<DSPARK_GREEDY, kEpiRow, true>(p) : pick3<DSPARK_GREEDY, kEpiRow, false>(p);
}

}  // namespace dspark
