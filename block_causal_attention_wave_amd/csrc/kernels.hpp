// Launch interfaces of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace wave {

// One round's K/V write.  `writes` points at the round's rows of the write
// table in the device descriptor (phys_slot, len, src_offset, 0 per row).
struct KvWriteArgs {
  const int32_t* writes;
  int32_t num_writes;
  void* k;
  void* vt;
  int32_t heads, head_dim, lpad;
  const void* k_src;
  const void* v_src;
  int32_t src_fp32;
  int64_t src_row_stride;  // elements
};

// One round's attention.  Table pointers are the descriptor's node, ctx and
// work tables; the round's items are work[work_begin .. work_begin+num_work).
struct AttnArgs {
  const int32_t* nodes;
  const int32_t* ctx;
  const int32_t* work;
  int32_t work_begin, num_work;
  const void* k;
  const void* vt;
  int32_t heads, head_dim, lpad;
  const void* q;
  int32_t q_fp32;
  int64_t q_row_stride;  // elements
  void* o;
  float* lse;
  int32_t lse_stride;  // rows of the round (LSE is [heads][rows])
  float scale_log2e;   // scale * log2(e)
  // split-KV: > 1 splits each node's key tiles into that many contiguous
  // ranges; partial results go to part_o (fp32 [splits][part_rows][heads][d])
  // and part_lse (fp32 [splits][heads][part_rows]) and are merged into o / lse.
  // Partial row = the round row (part_rows = the round's rows).
  int32_t num_splits;
  // Tail balancing (num_splits <= 1): items [0, num_direct) are processed
  // whole; each later item is cut into tail_splits key ranges, with partial
  // row = (item - num_direct) * 256 + row in the item (part_rows = the tail
  // items times 256), merged afterwards.  num_direct = num_work: none.
  int32_t num_direct;
  int32_t tail_splits;
  int32_t part_rows;
  float* part_o;
  float* part_lse;
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_wave_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace wave
