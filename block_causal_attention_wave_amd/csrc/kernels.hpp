// Launch interfaces of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace wave {

// Words per node row of the device descriptor: q_offset, q_len, ctx_begin,
// ctx_count, chunk, level.  A node's own slot is the last entry of its
// gather list.
constexpr int kDescNodeWords = 6;

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
  int32_t stream_out;      // non-temporal cache stores (see launch_kv_write)
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
  // Optional (nullptr: none): fp32 [rows][heads], per output row and head
  // the sum of squares of the row's bf16 O values over head_dim (the next
  // layer's RMS statistics in the toy chain).
  float* row_sq;
};

// Output tile of one qkv_project workgroup: tokens x projection columns.
constexpr int kProjTileRows = 256, kProjTileCols = 128;

// Toy-chain QKV projection of one round at one layer: every node's input
// rows x (round-packed [round rows][D], or per-chunk state [chunks][chunk_rows][D]
// when x_chunk) times W^T ([3D][D]), scaled per row by 1/rms (row_scale,
// indexed by round row), to Q (round-packed [rows][D]) and the node's own
// K / V^T cache slot.  Workgroups: (node, row tile, column tile).
struct ProjArgs {
  const int32_t* nodes;
  const int32_t* ctx;
  int32_t node_begin, num_nodes, max_rows, row_tiles, col_tiles;
  const void* x;
  int32_t x_chunk, chunk_rows;
  const void* w;
  int32_t model_dim, heads, head_dim, lpad;
  void* k;
  void* vt;
  void* q;
  float* row_scale;
  // Optional (nullptr: 1/rms computed from x into row_scale first): fp32
  // [round rows][heads] sums of squares of x's rows per head, as wave_attn
  // writes them for its O; x must then be the round-packed O.
  const float* row_sq;
};

// Copy of each node's output rows o[q_offset ..] to its chunk's state rows.
struct StoreArgs {
  const int32_t* nodes;
  int32_t node_begin, num_nodes, max_rows, model_dim, chunk_rows;
  const void* o;
  void* state;
};

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_qkv_project(const ProjArgs& a, hipStream_t stream);
hipError_t launch_chain_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_wave_attn(const AttnArgs& a, hipStream_t stream);

// Size of the per-device scratch array behind the allocation-free split-KV
// entry point, and the lookup of the current device's copy (its device
// address, found once per device and kept).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_buffer(void** ptr);

}  // namespace wave
