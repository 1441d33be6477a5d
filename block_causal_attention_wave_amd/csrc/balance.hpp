// Tail balancing of one attention round (host side).
//
// wave_attn runs one workgroup per (work item, head), items in the plan's
// order: most key tiles first.  The hardware hands workgroups to compute
// units in launch order, so when their count is not a multiple of the units
// the last ones run on a part-empty chip.  Cutting the key ranges of the last
// few items into pieces (merged by a second, small kernel) evens out the
// finish.  The choice below comes from simulating that in-order dispatch.
#pragma once

#include <cstdint>

#include "planner.hpp"

namespace wave {

struct TailSplit {
  int32_t items = 0;   // trailing work items of the round cut into pieces
  int32_t splits = 1;  // pieces per item (contiguous key-tile ranges)
};

// Best split of the last items of `round` for `heads` heads of `head_dim`
// on `cus` compute units, counting the merge pass (items = 0 when no split
// shortens the simulated round).
TailSplit choose_tail_split(const Plan& p, int32_t round, int32_t heads, int32_t head_dim, int32_t cus);

// Key splits for split-KV attention of `round` (every work item cut into
// that many ranges), 1..64: the most that still fit the round's workgroups
// (items x heads x splits) onto the `cus` compute units in one dispatch wave,
// at most the longest item's key-tile count.
int32_t choose_splits(const Plan& p, int32_t round, int32_t heads, int32_t head_dim, int32_t cus);

// Simulated duration, in key-tile times, of the round with that split: each
// workgroup costs its key tiles plus a fixed start-up; pieces pay a partial
// result write as well.  The merge pass is not included.
double simulate_round(const Plan& p, int32_t round, int32_t heads, int32_t cus, const TailSplit& t);

}  // namespace wave
