// qkv_project and chain_store: the steps on either side of the attention in
// the toy denoiser chain, on gfx950.
//
// The pages carry no model, so a seeded stand-in closes the loop between
// denoising levels: a chunk's next node consumes its previous node's output
// (Wave Forcing summary, mechanism paragraph; design-space paper, Figure 2),
// and every node projects its input to Q, K and V.  Per layer:
//   [Q | K | V] = bf16( (A W^T) / rms(A) ),  rms(a) = sqrt(mean_c a_c^2 + 1e-6)
// with A the node's input rows [L][D] (D = heads * head_dim) and W [3D][D].
// The K and V columns go straight into the node's own cache slot (K
// token-major, V transposed, zero past the chunk's tokens), so no separate
// K/V copy pass is needed; Q goes to the round's packed query rows.
//
// Kernels:
//   row_scale_kernel  1 / rms of every input row (one wave per row); or
//   row_scale_from_sq_kernel  the same from per-head sums of squares of the
//                     rows that the attention wrote with its O (wave_attn_chain).
//   qkv_gemm_kernel   one workgroup per (node, 256-token tile, 128-column
//                     tile), 8 waves of 64x64: bf16 MFMA 32x32x16, fp32
//                     accumulation, a three-stage LDS ring of 256x64 A and
//                     128x64 W tiles filled by direct global->LDS loads (two
//                     k-steps in flight, one barrier per k-step), and an
//                     epilogue that scales, rounds and scatters the tile
//                     through LDS.
//   qkv_gemm_wide_kernel  the same with 256-column tiles (8 waves of 128x64,
//                     two 64 KiB stages), for model dims that are multiples
//                     of 256: fewer operand reads and tile bytes per flop.
//   chain_store_kernel  copies each node's output rows to its chunk's state.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace wave {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = kProjTileRows, TN = kProjTileCols, TK = 64;
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int NSTAGE = 3;
constexpr int ROW_BYTES = TK * 2;              // one tile row in LDS
constexpr int A_BYTES = TM * ROW_BYTES;        // 32 KiB
constexpr int W_BYTES = TN * ROW_BYTES;        // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + W_BYTES;  // A tile then W tile
constexpr int A_LOADS = A_BYTES / (THREADS * 16);  // 16-byte loads per thread per A tile
constexpr int W_LOADS = W_BYTES / (THREADS * 16);
constexpr int OUT_PITCH_R = (TN + 8) * 2;      // row-major staging: bytes per token row
constexpr int OUT_PITCH_C = (TM + 8) * 2;      // column-major staging: bytes per column
static_assert(TM == 4 * 64 && TN == 2 * 64, "8 waves of 64x64");
static_assert(TM * OUT_PITCH_R <= NSTAGE * STAGE_BYTES && TN * OUT_PITCH_C <= NSTAGE * STAGE_BYTES,
              "the staged output tile fits in the ring");

// 16-byte chunk swizzle of a 128-byte LDS row: a 16-byte LDS read is served
// 16 lanes at a time (a half-wave's lane quads of equal index parity), and an
// MFMA operand read puts consecutive lanes on consecutive rows at one chunk.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// 1 / rms of each input row of the round's nodes: grid (row blocks, nodes),
// one wave per row.
__global__ __launch_bounds__(256) void row_scale_kernel(ProjArgs a) {
  const int node = a.node_begin + blockIdx.y;
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], L = nd[1], chunk = nd[4];
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= L) return;
  const int64_t src_row = (a.x_chunk ? (int64_t)chunk * a.chunk_rows : (int64_t)q_offset) + r;
  const bf16x8* row = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.x) + src_row * a.model_dim);
  float ss = 0.0f;
  for (int c = lane; c < a.model_dim / 8; c += 64) {
    const bf16x8 v = row[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf((float)v[i], (float)v[i], ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) a.row_scale[q_offset + r] = 1.0f / __builtin_sqrtf(ss / (float)a.model_dim + 1e-6f);
}

// The same 1 / rms from per-head sums of squares of the rows (as
// wave_attn_chain writes them for its O, which is then x): one thread per
// row, grid (row blocks, nodes).
__global__ __launch_bounds__(256) void row_scale_from_sq_kernel(ProjArgs a) {
  const int node = a.node_begin + blockIdx.y;
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], L = nd[1];
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= L) return;
  const float* sq = a.row_sq + (int64_t)(q_offset + r) * a.heads;
  // four independent chains, so that the loads of a group issue together
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int h = 0;
  for (; h + 4 <= a.heads; h += 4) {
    s0 += sq[h];
    s1 += sq[h + 1];
    s2 += sq[h + 2];
    s3 += sq[h + 3];
  }
  for (; h < a.heads; ++h) s0 += sq[h];
  const float ss = (s0 + s1) + (s2 + s3);
  a.row_scale[q_offset + r] = 1.0f / __builtin_sqrtf(ss / (float)a.model_dim + 1e-6f);
}

template <int HD>
__global__ __launch_bounds__(THREADS, 2) void qkv_gemm_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wv >> 1, wc = wv & 1;  // this wave's 64x64 block of the tile
  // Tile order.  The dispatcher hands workgroup i to XCD i % 8; each XCD has
  // its own L2.  Remap so that every XCD runs a contiguous range of tiles,
  // and within a node order them by groups of 4 row tiles x all column
  // tiles (row tile fastest): the ~32 workgroups an XCD runs at once then
  // cover 4 A row tiles x 8 W column tiles and share their k-slices in L2.
  int b = blockIdx.x;
  {
    const int per_xcd = (int)(gridDim.x / 8);
    if (b < per_xcd * 8) b = (b % 8) * per_xcd + b / 8;
  }
  const int per_node = a.row_tiles * a.col_tiles;
  const int node = a.node_begin + b / per_node;
  int rt, ct;
  {
    constexpr int G = 4;
    const int r = b % per_node;
    const int full = a.row_tiles / G;
    const int gsz = G * a.col_tiles;
    if (r < full * gsz) {
      ct = (r % gsz) / G;
      rt = (r / gsz) * G + r % G;
    } else {
      const int rem = a.row_tiles - full * G, rr = r - full * gsz;
      ct = rr / rem;
      rt = full * G + rr % rem;
    }
  }
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], L = nd[1], chunk = nd[4];
  const int phys = a.ctx[2 * (nd[2] + nd[3] - 1)];  // the node's own slot: last in its gather list
  const int D = a.model_dim;
  const int r0 = rt * TM, c0 = ct * TN;

  // Per-lane byte offsets of this thread's tile loads (A rows past the
  // chunk's tokens re-read its last row; their results are dropped).
  const char* abase = static_cast<const char*>(a.x) +
                      ((a.x_chunk ? (int64_t)chunk * a.chunk_rows : (int64_t)q_offset) * D) * 2;
  const char* wbase = static_cast<const char*>(a.w) + (int64_t)c0 * D * 2;
  uint32_t aoff[A_LOADS], woff[W_LOADS];
#pragma unroll
  for (int n = 0; n < A_LOADS; ++n) {
    const int off = (wv * A_LOADS + n) * 1024 + lane * 16;
    const int row = off / ROW_BYTES;
    const int lc = ((off % ROW_BYTES) / 16) ^ swz(row);
    aoff[n] = (uint32_t)(((int64_t)min(r0 + row, L - 1) * D + lc * 8) * 2);
  }
#pragma unroll
  for (int n = 0; n < W_LOADS; ++n) {
    const int off = (wv * W_LOADS + n) * 1024 + lane * 16;
    const int row = off / ROW_BYTES;
    const int lc = ((off % ROW_BYTES) / 16) ^ swz(row);
    woff[n] = (uint32_t)(((int64_t)row * D + lc * 8) * 2);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int ks, int stage) {
    const char* ab = abase + (int64_t)ks * TK * 2;
    const char* wb = wbase + (int64_t)ks * TK * 2;
    const uint32_t sa = lds0 + stage * STAGE_BYTES, sw = sa + A_BYTES;
#pragma unroll
    for (int n = 0; n < A_LOADS; ++n) load_lds16(sa + (wv * A_LOADS + n) * 1024, ab, aoff[n]);
#pragma unroll
    for (int n = 0; n < W_LOADS; ++n) load_lds16(sw + (wv * W_LOADS + n) * 1024, wb, woff[n]);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int kWaitExp = (0x7 << 4) | (0xF << 8);  // wait on vmcnt only

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Three-stage ring: k-steps ks and ks+1 in flight while ks is consumed;
  // k-step ks+2 goes into the stage k-step ks-1 used, after the barrier that
  // every wave passes only once done with ks-1.
  const int nk = D / TK;
  constexpr int TILE_LOADS = A_LOADS + W_LOADS;
  static_assert(TILE_LOADS <= 15, "vmcnt immediate");
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  int stage = 0;
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) __builtin_amdgcn_s_waitcnt(kWaitExp | TILE_LOADS);  // k-step ks has landed
    else __builtin_amdgcn_s_waitcnt(kWaitExp);
    barrier();
    if (ks + 2 < nk) issue(ks + 2, stage == 0 ? 2 : stage - 1);
    const char* sa = lds + stage * STAGE_BYTES;
    const char* sw = sa + A_BYTES;
    // Operand fragments of 16-deep substep s+1 are read while the MFMAs of
    // substep s run.
    auto frags = [&](int s, bf16x8 (&af)[2], bf16x8 (&bf)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wr * 64 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(sa + row * ROW_BYTES + (((2 * s + (lane >> 5)) ^ swz(row)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wc * 64 + j * 32 + (lane & 31);
        bf[j] = *reinterpret_cast<const bf16x8*>(sw + row * ROW_BYTES + (((2 * s + (lane >> 5)) ^ swz(row)) * 16));
      }
    };
    bf16x8 af[2][2], bf[2][2];
    frags(0, af[0], bf[0]);
#pragma unroll
    for (int s = 0; s < TK / 16; ++s) {
      if (s + 1 < TK / 16) frags(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
    }
    // Keep that order: reads of substeps 0 and 1, then (MFMAs of s, reads of s+2).
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int s = 0; s < TK / 16 - 2; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    stage = stage == NSTAGE - 1 ? 0 : stage + 1;
  }
  barrier();  // the epilogue reuses the ring

  // Epilogue: scale rows by 1/rms (0 past the chunk's tokens), round to bf16
  // and stage the tile in LDS: row-major for Q and K columns, column-major
  // (tokens contiguous) for V columns.
  const int part = c0 / D;  // 0: Q, 1: K, 2: V (D is a multiple of TN)
  // MFMA 32x32 accumulator: register e of lane l is row 8(e/4) + 4(l/32) + e%4, column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row0 = wr * 64 + i * 32 + 8 * g + 4 * (lane >> 5);
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + row0 + e;
        sc[e] = r < L ? a.row_scale[q_offset + r] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wc * 64 + j * 32 + (lane & 31);
        if (part == 2) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[i][j][4 * g + e] * sc[e]);
          *reinterpret_cast<bf16x4*>(lds + col * OUT_PITCH_C + row0 * 2) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            *reinterpret_cast<__bf16*>(lds + (row0 + e) * OUT_PITCH_R + col * 2) = (__bf16)(acc[i][j][4 * g + e] * sc[e]);
        }
      }
    }
  }
  __syncthreads();
  const int heads = a.heads, lpad = a.lpad;
  for (int id = tid; id < TM * (TN / 8); id += THREADS) {
    if (part == 2) {
      const int col = id / (TM / 8), tok = r0 + (id % (TM / 8)) * 8;
      if (tok >= lpad) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + col * OUT_PITCH_C + (tok - r0) * 2);
      const int h = (c0 - 2 * D + col) / HD, dd = (c0 - 2 * D + col) % HD;
      __bf16* dst = static_cast<__bf16*>(a.vt) + (((int64_t)phys * heads + h) * HD + dd) * lpad + tok;
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      const int row = id / (TN / 8), cc = (id % (TN / 8)) * 8;
      const int r = r0 + row;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * OUT_PITCH_R + cc * 2);
      if (part == 0) {
        if (r >= L) continue;
        __bf16* dst = static_cast<__bf16*>(a.q) + (int64_t)(q_offset + r) * D + c0 + cc;
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        if (r >= lpad) continue;
        const int h = (c0 - D + cc) / HD, dd = (c0 - D + cc) % HD;
        __bf16* dst = static_cast<__bf16*>(a.k) + (((int64_t)phys * heads + h) * lpad + r) * HD + dd;
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
}

// Wide tiles, for model dims that are multiples of 256: one workgroup per
// (node, 256-token tile, 256-column tile), 8 waves of 128x64.  Per 16-deep
// substep a wave reads 6 operand fragments for 8 MFMAs (4 for 4 above), and
// a tile loads 128 bytes of A and W per 256 * 256 * 2 flops (against 192).
// Two 64 KiB stages: k-step ks+1 streams in while ks is multiplied.
namespace wide {
constexpr int TM = 256, TN = 256, TK = 64, NSTAGE = 2;
constexpr int ROW_BYTES = TK * 2;
constexpr int A_BYTES = TM * ROW_BYTES;
constexpr int W_BYTES = TN * ROW_BYTES;
constexpr int STAGE_BYTES = A_BYTES + W_BYTES;
constexpr int A_LOADS = A_BYTES / (THREADS * 16);
constexpr int W_LOADS = W_BYTES / (THREADS * 16);
constexpr int OUT_PITCH_R = (TN + 8) * 2;
constexpr int OUT_PITCH_C = (TM + 8) * 2;
constexpr int LDS_BYTES = TM * OUT_PITCH_R > NSTAGE * STAGE_BYTES ? TM * OUT_PITCH_R : NSTAGE * STAGE_BYTES;
static_assert(TN * OUT_PITCH_C <= LDS_BYTES, "column-major staging fits");
static_assert(A_LOADS + W_LOADS <= 15, "vmcnt immediate");
}  // namespace wide

template <int HD>
__global__ __launch_bounds__(THREADS, 1) void qkv_gemm_wide_kernel(ProjArgs a) {
  using wide::TM;
  using wide::TN;
  using wide::TK;
  using wide::ROW_BYTES;
  using wide::A_BYTES;
  using wide::STAGE_BYTES;
  using wide::A_LOADS;
  using wide::W_LOADS;
  using wide::OUT_PITCH_R;
  using wide::OUT_PITCH_C;
  __shared__ __attribute__((aligned(1024))) char lds[wide::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wv >> 2, wc = wv & 3;  // this wave's 128x64 block of the tile
  // Tile order as in qkv_gemm_kernel: contiguous tile ranges per XCD, groups
  // of 4 row tiles x all column tiles inside a node.  When a node's last row
  // tile holds at most 128 rows of the slot (lpad), those tiles, whose
  // second half of waves skips the arithmetic, go last: they fill the
  // dispatch's final, part-empty wave at about half the cost of a full tile.
  const int last_rows = a.lpad - (a.row_tiles - 1) * TM;
  const int tail = a.row_tiles > 1 && last_rows <= TM / 2 ? 1 : 0;
  const int body_rows = a.row_tiles - tail;
  const int body = a.num_nodes * body_rows * a.col_tiles;
  auto xcd_order = [](int b, int n) {  // workgroup b of n -> tile index, one contiguous range per XCD
    const int per_xcd = n / 8;
    return b < per_xcd * 8 ? (b % 8) * per_xcd + b / 8 : b;
  };
  int node, rt, ct;
  if ((int)blockIdx.x < body) {
    const int b = xcd_order(blockIdx.x, body);
    const int per_node = body_rows * a.col_tiles;
    node = a.node_begin + b / per_node;
    constexpr int G = 4;
    const int r = b % per_node;
    const int full = body_rows / G;
    const int gsz = G * a.col_tiles;
    if (r < full * gsz) {
      ct = (r % gsz) / G;
      rt = (r / gsz) * G + r % G;
    } else {
      const int rem = body_rows - full * G, rr = r - full * gsz;
      ct = rr / rem;
      rt = full * G + rr % rem;
    }
  } else {
    const int b = xcd_order((int)blockIdx.x - body, (int)gridDim.x - body);
    node = a.node_begin + b / a.col_tiles;
    ct = b % a.col_tiles;
    rt = a.row_tiles - 1;
  }
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], L = nd[1], chunk = nd[4];
  const int phys = a.ctx[2 * (nd[2] + nd[3] - 1)];  // the node's own slot: last in its gather list
  const int D = a.model_dim;
  const int r0 = rt * TM, c0 = ct * TN;
  // waves whose 128 rows all lie past the slot's end only help load and sync
  const bool active = r0 + wr * 128 < a.lpad;

  const char* abase = static_cast<const char*>(a.x) +
                      ((a.x_chunk ? (int64_t)chunk * a.chunk_rows : (int64_t)q_offset) * D) * 2;
  const char* wbase = static_cast<const char*>(a.w) + (int64_t)c0 * D * 2;
  uint32_t aoff[A_LOADS], woff[W_LOADS];
#pragma unroll
  for (int n = 0; n < A_LOADS; ++n) {
    const int off = (wv * A_LOADS + n) * 1024 + lane * 16;
    const int row = off / ROW_BYTES;
    const int lc = ((off % ROW_BYTES) / 16) ^ swz(row);
    aoff[n] = (uint32_t)(((int64_t)min(r0 + row, L - 1) * D + lc * 8) * 2);
  }
#pragma unroll
  for (int n = 0; n < W_LOADS; ++n) {
    const int off = (wv * W_LOADS + n) * 1024 + lane * 16;
    const int row = off / ROW_BYTES;
    const int lc = ((off % ROW_BYTES) / 16) ^ swz(row);
    woff[n] = (uint32_t)(((int64_t)row * D + lc * 8) * 2);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int ks, int stage) {
    const char* ab = abase + (int64_t)ks * TK * 2;
    const char* wb = wbase + (int64_t)ks * TK * 2;
    const uint32_t sa = lds0 + stage * STAGE_BYTES, sw = sa + A_BYTES;
#pragma unroll
    for (int n = 0; n < A_LOADS; ++n) load_lds16(sa + (wv * A_LOADS + n) * 1024, ab, aoff[n]);
#pragma unroll
    for (int n = 0; n < W_LOADS; ++n) load_lds16(sw + (wv * W_LOADS + n) * 1024, wb, woff[n]);
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int kWaitExp = (0x7 << 4) | (0xF << 8);  // wait on vmcnt only

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Q and K tiles are multiplied transposed (W rows as the MFMA's A operand,
  // token rows as B), so that each lane ends with 4 consecutive columns of
  // one token and the row-major staging below takes 8-byte writes; V tiles
  // keep tokens consecutive in a lane for the column-major (V^T) staging.
  const int part = c0 / D;  // 0: Q, 1: K, 2: V (D is a multiple of TN)
  // 1/rms of token (lane & 31) of each of the wave's 32-token blocks (0 past
  // the chunk's tokens), fetched now so that the epilogue does not wait.
  // With per-head sums of squares (x = the attention's O that wrote them),
  // the tile's 256 scales are formed here instead, after the first tile's
  // loads are issued, and kept in LDS: two threads per row, one of every
  // other head each.
  __shared__ float rs_lds[TM];
  const bool from_sq = a.row_sq != nullptr;
  float rsc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (!from_sq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + wr * 128 + i * 32 + (lane & 31);
      rsc[i] = r < L ? a.row_scale[q_offset + r] : 0.0f;
    }
  }
  auto scales_from_sq = [&]() __attribute__((always_inline)) {
    const int row = tid >> 1, hp = tid & 1;
    const int r = r0 + row;
    const float* sq = a.row_sq + (int64_t)(q_offset + min(r, L - 1)) * a.heads;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int h = hp + 2 * k;
      v[k] = h < a.heads ? sq[h] : 0.0f;
    }
    float ss = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    for (int h = hp + 16; h < a.heads; h += 2) ss += sq[h];
    ss += __shfl_xor(ss, 1, 64);
    if (hp == 0) rs_lds[row] = r < L ? 1.0f / __builtin_sqrtf(ss / (float)a.model_dim + 1e-6f) : 0.0f;
  };

  // Two stages: after the barrier of k-step ks every wave is done with ks-1,
  // whose stage receives ks+1 while ks is multiplied.
  const int nk = D / TK;
  auto kloop = [&](auto tr_tag) __attribute__((always_inline)) {
  constexpr bool TR = decltype(tr_tag)::value;
  issue(0, 0);
  if (from_sq) scales_from_sq();  // its loads' latency overlaps the first tile's; the k-loop's barriers publish it
  int stage = 0;
  for (int ks = 0; ks < nk; ++ks) {
    __builtin_amdgcn_s_waitcnt(kWaitExp);  // this thread's loads of k-step ks have landed
    barrier();
    if (ks + 1 < nk) issue(ks + 1, stage ^ 1);
    if (active) {
      const char* sa = lds + stage * STAGE_BYTES;
      const char* sw = sa + A_BYTES;
      auto frags = [&](int s, bf16x8 (&af)[4], bf16x8 (&bf)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wr * 128 + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8*>(sa + row * ROW_BYTES + (((2 * s + (lane >> 5)) ^ swz(row)) * 16));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = wc * 64 + j * 32 + (lane & 31);
          bf[j] = *reinterpret_cast<const bf16x8*>(sw + row * ROW_BYTES + (((2 * s + (lane >> 5)) ^ swz(row)) * 16));
        }
      };
      bf16x8 af[2][4], bf[2][2];
      frags(0, af[0], bf[0]);
#pragma unroll
      for (int s = 0; s < TK / 16; ++s) {
        if (s + 1 < TK / 16) frags(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
      }
      // Keep that order: reads of substeps 0 and 1, then (MFMAs of s, reads of s+2).
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
      for (int s = 0; s < TK / 16 - 2; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    stage ^= 1;
  }
  };
  if (part == 2) kloop(std::false_type{});
  else kloop(std::true_type{});
  barrier();  // the epilogue reuses the stages
  if (from_sq) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rsc[i] = rs_lds[wr * 128 + i * 32 + (lane & 31)];
  }

  // Epilogue: scale by 1/rms, round, stage in LDS (column-major for V), then
  // 16-byte stores to Q, K or V^T.  Q/K lanes hold token (lane & 31) of each
  // 32-token block and 4 consecutive columns per register quad.
  if (!active) {
    // rows past the slot's end: never written out
  } else if (part != 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wr * 128 + i * 32 + (lane & 31);
      const float sc = rsc[i];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wc * 64 + j * 32 + 8 * g + 4 * (lane >> 5);
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[i][j][4 * g + e] * sc);
          *reinterpret_cast<bf16x4*>(lds + row * OUT_PITCH_R + col * 2) = v;
        }
    }
  } else {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row0 = wr * 128 + i * 32 + 8 * g + 4 * (lane >> 5);
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = __shfl(rsc[i], 8 * g + 4 * (lane >> 5) + e, 64);  // lane t: token t
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wc * 64 + j * 32 + (lane & 31);
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[i][j][4 * g + e] * sc[e]);
        *reinterpret_cast<bf16x4*>(lds + col * OUT_PITCH_C + row0 * 2) = v;
      }
    }
  }
  }
  __syncthreads();
  // Write-out: every thread's 16 LDS reads first, then its 16-byte stores.
  const int heads = a.heads, lpad = a.lpad;
  constexpr int ITER = TM * (TN / 8) / THREADS;
  static_assert(ITER * THREADS == TM * (TN / 8), "whole write-out passes");
  u32x4 out[ITER];
  if (part == 2) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int id = tid + it * THREADS, col = id / (TM / 8), t8 = (id % (TM / 8)) * 8;
      out[it] = *reinterpret_cast<const u32x4*>(lds + col * OUT_PITCH_C + t8 * 2);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int id = tid + it * THREADS, col = id / (TM / 8), tok = r0 + (id % (TM / 8)) * 8;
      const int h = (c0 - 2 * D + col) / HD, dd = (c0 - 2 * D + col) % HD;
      if (tok < lpad)
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.vt) + (((int64_t)phys * heads + h) * HD + dd) * lpad + tok) =
            out[it];
    }
  } else {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int id = tid + it * THREADS, row = id / (TN / 8), cc = (id % (TN / 8)) * 8;
      out[it] = *reinterpret_cast<const u32x4*>(lds + row * OUT_PITCH_R + cc * 2);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int id = tid + it * THREADS, r = r0 + id / (TN / 8), cc = (id % (TN / 8)) * 8;
      if (part == 0) {
        if (r < L) *reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.q) + (int64_t)(q_offset + r) * D + c0 + cc) = out[it];
      } else if (r < lpad) {
        const int h = (c0 - D + cc) / HD, dd = (c0 - D + cc) % HD;
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.k) + (((int64_t)phys * heads + h) * lpad + r) * HD + dd) = out[it];
      }
    }
  }
}

// state[chunk rows] = o[node rows] for every node of the round: grid (row
// chunks of 256 x 8 elements, nodes).
__global__ __launch_bounds__(256) void chain_store_kernel(StoreArgs a) {
  const int node = a.node_begin + blockIdx.y;
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], L = nd[1], chunk = nd[4];
  const int64_t n16 = (int64_t)L * a.model_dim / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(a.o) + (int64_t)q_offset * a.model_dim);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<__bf16*>(a.state) + (int64_t)chunk * a.chunk_rows * a.model_dim);
  dst[i] = src[i];
}

}  // namespace

hipError_t launch_qkv_project(const ProjArgs& a, hipStream_t stream) {
  if (a.num_nodes == 0) return hipSuccess;
  const bool wide_tiles = a.model_dim % wide::TN == 0;
  if (a.row_sq == nullptr) {
    dim3 sgrid((unsigned)((a.max_rows + 3) / 4), (unsigned)a.num_nodes);
    hipLaunchKernelGGL(row_scale_kernel, sgrid, dim3(256), 0, stream, a);
  } else if (!wide_tiles) {  // the wide kernel forms the scales from row_sq itself
    dim3 sgrid((unsigned)((a.max_rows + 255) / 256), (unsigned)a.num_nodes);
    hipLaunchKernelGGL(row_scale_from_sq_kernel, sgrid, dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wide_tiles) {
    // 256-wide column tiles: a tile never straddles the Q / K / V parts
    ProjArgs w = a;
    w.col_tiles = 3 * a.model_dim / wide::TN;
    dim3 grid((unsigned)(w.num_nodes * w.row_tiles * w.col_tiles));
    if (a.head_dim == 128) hipLaunchKernelGGL(qkv_gemm_wide_kernel<128>, grid, dim3(THREADS), 0, stream, w);
    else hipLaunchKernelGGL(qkv_gemm_wide_kernel<64>, grid, dim3(THREADS), 0, stream, w);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(a.num_nodes * a.row_tiles * a.col_tiles));
  if (a.head_dim == 128) hipLaunchKernelGGL(qkv_gemm_kernel<128>, grid, dim3(THREADS), 0, stream, a);
  else hipLaunchKernelGGL(qkv_gemm_kernel<64>, grid, dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_chain_store(const StoreArgs& a, hipStream_t stream) {
  if (a.num_nodes == 0) return hipSuccess;
  const int64_t n16 = (int64_t)a.max_rows * a.model_dim / 8;
  dim3 grid((unsigned)((n16 + 255) / 256), (unsigned)a.num_nodes);
  hipLaunchKernelGGL(chain_store_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wave
