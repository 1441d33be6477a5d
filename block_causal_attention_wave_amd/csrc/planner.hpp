// Host-side wave planner: (chunk, level) node DAG, round packing, physical
// cache slot allocation and the packed device descriptor.  Plain C++17, no
// HIP dependency.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "wave.h"

namespace wave {

// Descriptor layout (int32 words).  Header:
//   [0] magic, [1] version, [2..6] counts (rounds, nodes, ctx, writes, work),
//   [7..11] word offsets of the round, node, ctx, write and work tables.
// Tables (one row per element, fixed stride):
//   round : node_begin, node_end, write_begin, write_end, work_begin, work_end, q_rows, src_rows
//   node  : q_offset, q_len, ctx_begin, ctx_count, chunk, level
//   ctx   : phys_slot, len
//   write : phys_slot, len, src_offset, 0
//   work  : node, q_start, q_rows, 0
constexpr int32_t kDescMagic = 0x57415645;  // "WAVE"
constexpr int32_t kDescVersion = 2;
constexpr int kRoundStride = 8, kNodeStride = 6, kCtxStride = 2, kWriteStride = 4, kWorkStride = 4;
constexpr int kDescHeader = 12;

struct Plan {
  wave_plan_params params{};
  int32_t num_phys_slots = 0;
  int32_t max_slot_len = 0;
  int32_t max_ctx = 0;
  std::vector<int32_t> round_node_begin, round_write_begin, round_work_begin;
  std::vector<int32_t> round_q_rows, round_src_rows;
  std::vector<wave_node> nodes;
  std::vector<wave_slot_ref> ctx, writes;
  std::vector<wave_work> work;
  std::vector<int32_t> desc;  // packed descriptor
  int32_t num_rounds() const { return static_cast<int32_t>(round_q_rows.size()); }
};

// Builds a plan; returns WAVE_OK or an error code with *err set.
int32_t build_plan(const wave_plan_params& p, Plan& out, std::string* err);

}  // namespace wave
