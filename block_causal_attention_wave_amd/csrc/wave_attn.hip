// wave_attn: block-causal flash attention of one wave round on gfx950.
//
// Each query chunk of the round attends to its own tokens (both directions)
// and to the earlier chunks' K/V its context policy selects (streaming video
// diffusion design-space paper, arXiv 2609.22283 listing, Figure 1 and
// Table 1; Wave Forcing summary on aiany.app, mechanism paragraph; Wan-Streamer
// v0.2, Figure 1: block-causal attention on one timeline).  The mask is never
// materialised: every node carries a gather list of the cache slots it may
// read, and the kernel streams exactly those slots' key tiles.  The only
// masking left is the ragged tail of a slot's last tile.
//
// Work decomposition: one workgroup = 256 query rows of one node and one
// head; W waves of 32*QB query rows each.  Key tiles of 64 keys stream through
// a 4-stage LDS ring filled by direct global->LDS 16-byte loads issued by all
// waves; one barrier per tile.
//
// Contraction layout (bf16 MFMA 32x32x16, fp32 accumulation):
//   S^T[key][query] = K . Q^T   A = K rows from LDS, B = Q from registers.
//     With keys on the MFMA row axis, one lane holds one query and 16 keys,
//     so the softmax row max and row sum are in-lane except one exchange
//     between the two half-waves.  The K rows are stored permuted in LDS so
//     that a lane's 16 accumulator registers are 16 consecutive keys.
//   O^T[d][query] += V^T . P^T  A = V^T rows from LDS, B = P straight from the
//     softmax registers (bf16), no data movement.
// Online softmax in fp32: exp2 with the scale folded into one FMA, deferred
// 1/l normalisation (FlashAttention-2), and a lazily raised reference: the
// first block sets it to the exact row max, and it only moves again (with an
// O and l rescale) when a block's probabilities, formed against it, sum to
// more than 2^8 in some lane.  The common block computes no row max at all.
// Each 32-key step issues the next block's scores and the previous block's
// P.V product on the matrix cores and forms the current block's
// probabilities on the vector ALUs, interleaved in one instruction stream;
// with two waves per SIMD the hardware interleaves them as well, and the
// two waves take turns, tile by tile, at the higher issue priority.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace wave {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKT = 64;       // keys per LDS tile
constexpr int kStages = 4;    // LDS ring depth
constexpr int kMaxCtx = 512;  // gather-list entries staged in LDS
constexpr int kQTile = 256;   // query rows per workgroup

// W waves, QB 32-query blocks per wave, head dim HD.
template <int HD, int W, int QB>
struct Cfg {
  static constexpr int THREADS = 64 * W;
  static constexpr int KROW = HD * 2;  // bytes per K row in LDS
  static constexpr int KBYTES = kKT * KROW;
  static constexpr int VROW = kKT * 2;  // bytes per V^T row in LDS
  static constexpr int VBYTES = HD * VROW;
  static constexpr int VBASE = 4 * KBYTES;  // K tiles of all stages, then V^T tiles
  static constexpr int NC = HD / 16;  // k-steps of Q.K^T
  static constexpr int ND = HD / 32;  // d blocks of O^T
  static constexpr int KLOADS = KBYTES / (THREADS * 16);
  static constexpr int VLOADS = VBYTES / (THREADS * 16);
  static constexpr int LOADS = KLOADS + VLOADS;
  static_assert(W * 32 * QB == kQTile, "a workgroup covers one query tile");
  static_assert(KLOADS >= 1 && VLOADS >= 1, "every thread loads part of each tile");
};

// 16-byte chunk swizzles inside an LDS row.  gfx950 serves a 16-byte-per-lane
// LDS read 16 lanes at a time over 64 four-byte banks: one half-wave, and in
// it the four lane quads whose index ((lane >> 2) & 7) has the same bit
// parity.  An MFMA operand read puts the 32 lanes of a half-wave on 32
// consecutive rows at one logical chunk; these swizzles give the 16 lanes of
// every service group distinct banks.
__device__ __forceinline__ int swz16(int row) { return row & 15; }       // 256-byte rows
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }  // 128-byte rows
template <int HD>
__device__ __forceinline__ int swzK(int row) {
  if constexpr (HD == 128) return swz16(row);
  else return swz8(row);
}

// LDS row i of a K tile holds key perm_key(i): rows 32*kb + i' map so that the
// S^T accumulator of lane half h, register r, is key 32*kb + 16*h + r.
__device__ __forceinline__ int perm_key(int i) {
  const int kb = i >> 5, ip = i & 31;
  return kb * 32 + ((ip >> 2) & 1) * 16 + (ip >> 3) * 4 + (ip & 3);
}

// Per-lane byte offsets of one thread's share of a K/V tile load, relative
// to the tile's first key in the slot (the wave-uniform part of the address).
template <int HD, int W, int QB>
struct TileOffsets {
  using C = Cfg<HD, W, QB>;
  uint32_t k[C::KLOADS];
  uint32_t v[C::VLOADS];

  __device__ __forceinline__ TileOffsets(int lpad, int wv, int lane) {
#pragma unroll
    for (int n = 0; n < C::KLOADS; ++n) {
      const int off = (wv * C::KLOADS + n) * 1024 + lane * 16;
      const int row = off / C::KROW;
      const int lc = ((off % C::KROW) / 16) ^ swzK<HD>(row);
      k[n] = (uint32_t)((perm_key(row) * HD + lc * 8) * 2);
    }
#pragma unroll
    for (int n = 0; n < C::VLOADS; ++n) {
      const int off = (wv * C::VLOADS + n) * 1024 + lane * 16;
      const int d = off / C::VROW;
      const int lc = ((off % C::VROW) / 16) ^ swz8(d);
      v[n] = (uint32_t)((d * lpad + lc * 8) * 2);
    }
  }
};

// Issue one thread's direct global->LDS loads of a 64-key K tile (rows
// permuted, chunks swizzled) and the matching V^T tile.  kt / vt point at the
// tile's first key of the slot; wv is the (wave-uniform) wave index.  `stage`
// is the stage's K tile; its V^T tile sits VBASE bytes further.
template <int HD, int W, int QB>
__device__ __forceinline__ void issue_tile(char* stage, const char* kt, const char* vt,
                                           const TileOffsets<HD, W, QB>& off, int wv) {
  using C = Cfg<HD, W, QB>;
  const uint32_t kbase = (uint32_t)(uintptr_t)stage;
  const uint32_t vbase = kbase + C::VBASE;
#pragma unroll
  for (int n = 0; n < C::KLOADS; ++n)
    load_lds16(kbase + (wv * C::KLOADS + n) * 1024, kt, off.k[n]);
#pragma unroll
  for (int n = 0; n < C::VLOADS; ++n)
    load_lds16(vbase + (wv * C::VLOADS + n) * 1024, vt, off.v[n]);
}

// Row max / sum across the two half-waves (lanes l and l^32 hold the same query).
// The max helpers use the NaN-propagating IEEE maximum, which needs no
// quieting of its inputs (fmaxf does, at one extra instruction per element).
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float halfwave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halfwave_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw scores of one 32-key block (kb = 0 or 1 of a 64-key LDS tile) against
// the wave's 32*QB queries, as S^T blocks s[qb] (32 keys x 32 queries).
template <int HD, int QB>
__device__ __forceinline__ void qk_block(const char* ks, int kb, const bf16x8 (&qop)[QB][HD / 16],
                                         f32x16 (&s)[QB], int lane) {
  const int row = kb * 32 + (lane & 31);
  const char* rp = ks + row * (HD * 2);
  const int sw = swzK<HD>(row);
#pragma unroll
  for (int cc = 0; cc < HD / 16; ++cc) {
    const bf16x8 av = *reinterpret_cast<const bf16x8*>(rp + (((2 * cc + (lane >> 5)) ^ sw) * 16));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qop[qb][cc], cc == 0 ? f32x16{} : s[qb], 0, 0, 0);
  }
}

// Keys at or beyond `valid` (counted from the block's first key) get -inf.
// Called under a wave-uniform branch that is true for one block in ~70; the
// empty volatile asm keeps the compiler from if-converting the branch into
// per-element selects executed for every block.
template <int QB>
__device__ __forceinline__ void mask_block(f32x16 (&s)[QB], int valid, int lane) {
  asm volatile("");
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if ((lane >> 5) * 16 + r >= valid) s[qb][r] = -INFINITY;
}

__device__ __forceinline__ float block_rowmax(const f32x16& s) {
  // two independent chains of 3-input maxima
  float m0 = fmax_nan(fmax_nan(s[0], s[1]), s[2]);
  float m1 = fmax_nan(fmax_nan(s[3], s[4]), s[5]);
#pragma unroll
  for (int r = 6; r < 14; r += 4) {
    m0 = fmax_nan(fmax_nan(m0, s[r]), s[r + 1]);
    m1 = fmax_nan(fmax_nan(m1, s[r + 2]), s[r + 3]);
  }
  m0 = fmax_nan(fmax_nan(m0, s[14]), s[15]);
  return halfwave_max(fmax_nan(m0, m1));
}

// p = exp2(s * c2 - mref) (scores to log2 units and the softmax reference in
// one FMA), packed to bf16 MFMA B operands; the row sums accumulate the fp32
// probabilities (summing the bf16-rounded ones would cost the LSE up to 2^-9
// relative on short rows).
template <int QB>
__device__ __forceinline__ void softmax_block(const f32x16 (&s)[QB], float c2, const float (&mref)[QB],
                                              bf16x8 (&pop)[QB][2], float (&bsum)[QB]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float sum0 = 0.0f, sum1 = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 pv;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * hh + t], c2, -mref[qb]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 * hh + t + 1], c2, -mref[qb]));
        if (hh == 0 && t == 0) {
          sum0 = p0;
          sum1 = p1;
        } else {
          sum0 += p0;
          sum1 += p1;
        }
        pv[t] = (__bf16)p0;
        pv[t + 1] = (__bf16)p1;
      }
      pop[qb][hh] = pv;
    }
    bsum[qb] = sum0 + sum1;
  }
}

// O^T += V^T(block kb) . P^T
template <int HD, int QB>
__device__ __forceinline__ void pv_block(const char* vs, int kb, const bf16x8 (&pop)[QB][2],
                                         f32x16 (&o)[HD / 32][QB], int lane) {
#pragma unroll
  for (int db = 0; db < HD / 32; ++db) {
    const int d = db * 32 + (lane & 31);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int kc = 4 * kb + 2 * (lane >> 5) + hh;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(vs + d * (kKT * 2) + ((kc ^ swz8(d)) * 16));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pop[qb][hh], o[db][qb], 0, 0, 0);
    }
  }
}

// A block whose probabilities against the softmax reference sum to more than
// 2^kRescaleLog2 in some lane raises the reference (rescaling O and l);
// otherwise the stale reference is kept: each p <= 2^8 is exact enough in
// fp32 and bf16 and far from overflow in the fp32 accumulators.
constexpr float kRescaleLog2 = 8.0f;
constexpr float kRescaleSum = 256.0f;  // 2^kRescaleLog2

// Walks the gather list tile by tile, keeping the current slot's index and
// length in scalar registers.
struct Walker {
  const int* ctx;
  int count;
  int e = 0, t = 0, phys_ = 0, len_ = 0;
  __device__ __forceinline__ Walker(const int* c, int n) : ctx(c), count(n) { load(); }
  // Values read from LDS are per-lane to the compiler; they are the same in
  // every lane, and saying so keeps addresses and loop bounds in SGPRs.
  __device__ __forceinline__ void load() {
    if (e < count) {
      phys_ = __builtin_amdgcn_readfirstlane(ctx[2 * e]);
      len_ = __builtin_amdgcn_readfirstlane(ctx[2 * e + 1]);
    }
  }
  __device__ __forceinline__ int phys() const { return phys_; }
  __device__ __forceinline__ int key0() const { return t * kKT; }
  __device__ __forceinline__ int valid() const { return len_ - t * kKT; }  // >= kKT: full tile
  __device__ __forceinline__ void next() {
    if ((t + 1) * kKT >= len_) {
      ++e;
      t = 0;
      load();
    } else {
      ++t;
    }
  }
  // Advance k tiles, whole slots at a time.
  __device__ __forceinline__ void skip(int k) {
    while (k > 0 && e < count) {
      const int left = (len_ + kKT - 1) / kKT - t;
      if (k >= left) {
        k -= left;
        ++e;
        t = 0;
        load();
      } else {
        t += k;
        k = 0;
      }
    }
  }
};

// The loader's walk: the current tile's K and V^T addresses in scalar
// registers, stepped by one tile inside a slot and recomputed from the slot
// index when the walk enters the next slot.
template <int HD>
struct TileFeed {
  Walker w;
  const char* k0;  // K of this head in cache slot 0
  const char* v0;  // V^T of this head in cache slot 0
  int64_t slot_bytes;
  const char* kt = nullptr;
  const char* vt = nullptr;
  __device__ __forceinline__ TileFeed(const int* c, int n, const char* k, const char* v, int64_t sb, int first)
      : w(c, n), k0(k), v0(v), slot_bytes(sb) {
    w.skip(first);
    point();
  }
  __device__ __forceinline__ void point() {
    const int64_t off = (int64_t)w.phys() * slot_bytes;
    kt = k0 + off + (int64_t)w.key0() * (HD * 2);
    vt = v0 + off + (int64_t)w.key0() * 2;
  }
  __device__ __forceinline__ void next() {
    if ((w.t + 1) * kKT >= w.len_) {
      w.next();
      point();
    } else {
      ++w.t;
      kt += kKT * HD * 2;
      vt += kKT * 2;
    }
  }
};

// SPLIT = false: one workgroup per (work item, head) over the node's whole
// gather list; writes bf16 O and the LSE.  With tail balancing, the items
// after the first num_direct get tail_splits workgroups each, one per
// contiguous range of the node's key tiles, writing partial results (below).
// SPLIT = true (split-KV, for short query chunks against long contexts):
// one workgroup per (work item, head, key split) over a contiguous range of
// the node's key tiles.  Partial results are fp32 O normalised over the range
// and its LSE, merged afterwards by wave_attn_combine_kernel.  In split-KV
// mode and for work items shorter than a query tile, waves whose 32-row
// blocks hold no query row skip the arithmetic but keep loading tiles.
template <int HD, int W, int QB, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(W / 4, W / 4)))
void wave_attn_kernel(AttnArgs a) {
  using C = Cfg<HD, W, QB>;
  constexpr int NS = kStages;
  __shared__ __attribute__((aligned(1024))) char lds[NS * (C::KBYTES + C::VBYTES)];
  __shared__ int ctx_lds[2 * kMaxCtx];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wv_u = __builtin_amdgcn_readfirstlane(wv);
  int item, h, split = 0, nsplit = 1;
  bool partial = SPLIT;  // block-uniform: write partial results
  if constexpr (SPLIT) {
    const int hs = a.heads * a.num_splits;
    item = blockIdx.x / hs;
    h = (blockIdx.x % hs) / a.num_splits;
    split = blockIdx.x % a.num_splits;
    nsplit = a.num_splits;
  } else {
    const int direct = a.num_direct * a.heads;
    if ((int)blockIdx.x < direct) {
      item = blockIdx.x / a.heads;
      h = blockIdx.x % a.heads;
    } else {
      const int b = blockIdx.x - direct, hs = a.heads * a.tail_splits;
      item = a.num_direct + b / hs;
      h = (b % hs) / a.tail_splits;
      split = b % a.tail_splits;
      nsplit = a.tail_splits;
      partial = true;
    }
  }
  const int32_t* wk = a.work + 4 * (a.work_begin + item);
  const int node = wk[0], q_start = wk[1], q_rows = wk[2];
  const int32_t* nd = a.nodes + kDescNodeWords * node;
  const int q_offset = nd[0], ctx_count = nd[3];
  const int32_t* ctx_g = a.ctx + 2 * nd[2];
  // first partial row of this item (split-KV: its round row)
  const int64_t prow0 = SPLIT ? (int64_t)q_offset + q_start : (int64_t)(item - a.num_direct) * kQTile;

  // Two bodies: SKIP (split-KV, and work items shorter than a query tile)
  // lets waves whose 32-row blocks hold no query row skip the arithmetic;
  // full tiles run the body without that test.
  auto run = [&](auto skip_tag) __attribute__((always_inline)) {
    constexpr bool SKIP = decltype(skip_tag)::value;
    const int lpad = a.lpad;
    const int64_t slot_elems = (int64_t)a.heads * lpad * HD;
    const __bf16* kcache = static_cast<const __bf16*>(a.k) + (int64_t)h * lpad * HD;
    const __bf16* vcache = static_cast<const __bf16*>(a.vt) + (int64_t)h * HD * lpad;

    // The gather list goes to LDS once, so that walking it inside the tile
    // loop never waits on the vector-memory counter the K/V prefetch uses.
    for (int e = threadIdx.x; e < 2 * ctx_count; e += C::THREADS) ctx_lds[e] = ctx_g[e];
    // The V^T tile of ring stage NS-1 (where tile -1 would sit) starts as
    // zeros: the first pipeline step multiplies it by a zero P.
    for (int i = threadIdx.x; i < C::VBYTES / 16; i += C::THREADS)
      reinterpret_cast<f32x4*>(lds + C::VBASE + (kStages - 1) * C::VBYTES)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();
    int total_tiles = 0;
    for (int e = 0; e < ctx_count; ++e) total_tiles += (ctx_lds[2 * e + 1] + kKT - 1) / kKT;
    total_tiles = __builtin_amdgcn_readfirstlane(total_tiles);
    int first_tile = 0;
    if (partial) {
      const int per = (total_tiles + nsplit - 1) / nsplit;
      first_tile = min(total_tiles, split * per);
      total_tiles = min(total_tiles, first_tile + per) - first_tile;
      if (total_tiles <= 0) {  // empty range: weight zero in the merge
        for (int r = threadIdx.x; r < q_rows; r += C::THREADS)
          a.part_lse[((int64_t)split * a.heads + h) * a.part_rows + prow0 + r] = -INFINITY;
        return;
      }
    }
    const bool active = !SKIP || wv_u * QB * 32 < q_rows;  // wave-uniform (scalar compare)

    // Q fragments (B operand of S^T): lane holds query (lane & 31) of block qb,
    // dims 16c + 8*(lane>>5) .. +7.
    const float c2 = a.scale_log2e;
    bf16x8 qop[QB][C::NC];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r = (wv * QB + qb) * 32 + (lane & 31);
      const bool valid = r < q_rows;
      const int64_t base = (int64_t)(q_offset + q_start + r) * a.q_row_stride + (int64_t)h * HD + 8 * (lane >> 5);
  #pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        bf16x8 v;
        if (!valid) {
          for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
        } else if (a.q_fp32) {
          const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.q) + base + 16 * c);
          const f32x4 u = p[0], w = p[1];
          for (int i = 0; i < 4; ++i) {
            v[i] = (__bf16)u[i];
            v[4 + i] = (__bf16)w[i];
          }
        } else {
          v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + base + 16 * c);
        }
        qop[qb][c] = v;
      }
    }
    // Let the Q loads land here, on every path.  Their uses sit under
    // wave-uniform branches the compiler cannot see through, and it would
    // otherwise wait for every outstanding load (tile prefetches included)
    // before the first MFMA of each pipeline step.
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
      for (int c = 0; c < C::NC; ++c) asm volatile("" ::"v"(qop[qb][c]));

    f32x16 o[C::ND][QB];
  #pragma unroll
    for (int db = 0; db < C::ND; ++db)
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.0f;
    // Softmax reference per query in log2 units (c2 * a raw score): exact row
    // max of the first block, raised lazily afterwards.
    float mref[QB], l[QB];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] = 0.0f;

    TileFeed<HD> ld(ctx_lds, ctx_count, reinterpret_cast<const char*>(kcache),
                    reinterpret_cast<const char*>(vcache), slot_elems * 2, first_tile);
    const TileOffsets<HD, W, QB> toff(lpad, wv, lane);
    auto issue = [&](int stage) {
      issue_tile<HD, W, QB>(lds + stage * C::KBYTES, ld.kt, ld.vt, toff, wv_u);
      ld.next();
    };
    constexpr int kWaitExp = (0x7 << 4) | (0xF << 8);
    auto wait_tiles = [&](int later) {  // wait until at most `later` tiles of loads are in flight
      if (later >= 2) __builtin_amdgcn_s_waitcnt(kWaitExp | ((2 * C::LOADS) & 15) | (((2 * C::LOADS) >> 4) << 14));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(kWaitExp | (C::LOADS & 15) | ((C::LOADS >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(kWaitExp);
    };
    // Raw barrier: the wait above covers this thread's LDS fills, and the
    // compiler barriers keep LDS reads on their side of it.
    auto barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // Prologue: tiles 0..NS-2 in flight; scores of block 0 with an exact row max.
    for (int s = 0; s < NS - 1; ++s)
      if (s < total_tiles) issue(s);
    wait_tiles(min(total_tiles - 1, NS - 2));
    barrier();
    Walker cur(ctx_lds, ctx_count);
    cur.skip(first_tile);
    f32x16 sa[QB], sb[QB];
    if (active) {
      qk_block<HD, QB>(lds, 0, qop, sa, lane);
      if (cur.valid() < 32) mask_block<QB>(sa, cur.valid(), lane);
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) mref[qb] = c2 * block_rowmax(sa[qb]);
    }

    // A block's probabilities were formed against the current reference; if
    // some lane's sum over its 16 keys exceeds 2^kRescaleLog2 (a score above the
    // reference by more than that, or an overflow to inf), the block is redone:
    // its scores are recomputed from the K tile still in LDS, the reference is
    // raised to the block's exact row max (rescaling O and l), and the
    // probabilities are formed again.  Rare after the first block, which sets the
    // reference exactly; otherwise the block's sums go straight into l.
    auto settle = [&](float (&bsum)[QB], bf16x8 (&pop)[QB][2], const char* kst, int kb, int valid)
        __attribute__((always_inline)) {
      bool big = false;
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) big |= bsum[qb] > kRescaleSum;
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        f32x16 sr[QB];
        qk_block<HD, QB>(kst, kb, qop, sr, lane);
        if (valid < 32) mask_block<QB>(sr, valid, lane);
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float delta = fmaxf(c2 * block_rowmax(sr[qb]) - mref[qb], 0.0f);
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          mref[qb] += delta;
          l[qb] *= alpha;
  #pragma unroll
          for (int db = 0; db < C::ND; ++db)
  #pragma unroll
            for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
        }
        softmax_block<QB>(sr, c2, mref, pop, bsum);
      }
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) l[qb] += bsum[qb];
    };

    // Software pipeline over 32-key blocks: step j issues the scores of block
    // j+1 and the P.V product of block j-1 on the matrix cores, then forms the
    // probabilities of block j on the vector ALUs; the three are independent,
    // so one wave's MFMA and VALU work overlap.  Block j's P waits in
    // registers (pprev) until step j+1.  Each 64-key tile is two steps (block 0
    // with scores in sa, block 1 with scores in sb); the ring stage of tile n is
    // n % NS and the loop is unrolled NS tiles so that every LDS operand address
    // is a per-lane base plus an immediate.
    // The V^T region starts at 64 KiB, past the reach of an LDS instruction's
    // immediate offset; hiding its start from the compiler makes it part of the
    // per-lane base register, so the stage and block offsets stay immediates.
    uint32_t vregion = C::VBASE;
    asm volatile("" : "+s"(vregion));
    bf16x8 pprev[QB][2];
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb)
  #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
  #pragma unroll
        for (int i = 0; i < 8; ++i) pprev[qb][hh][i] = (__bf16)0.0f;
    auto step = [&](int n, auto stage_tag, auto kb_tag, f32x16 (&scur)[QB], f32x16 (&snext)[QB])
        __attribute__((always_inline)) {
      constexpr int ST = decltype(stage_tag)::value;
      constexpr int KB = decltype(kb_tag)::value;
      constexpr int SP = (ST + NS - 1) % NS;  // stage of tile n-1
      const char* kst = lds + ST * C::KBYTES;
      const char* vst = lds + vregion + ST * C::VBYTES;
      // Issue priority alternates tile by tile between the two waves that
      // share a SIMD (waves w and w+4).  At equal priority the older wave
      // always wins, runs ahead, and then idles at the tile barrier while
      // the younger one finishes alone without a partner to overlap with.
      if constexpr (KB == 0) {
        if (((wv_u >> 2) ^ n) & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      const int valid = cur.valid();
      const bool has_next = KB == 0 || n + 1 < total_tiles;
      if constexpr (KB == 1) {
        wait_tiles(min(total_tiles - 2 - n, NS - 3));
        barrier();
        if (n + NS - 1 < total_tiles) issue((ST + NS - 1) % NS);
      }
      if (active) {
        // Without a next block the scores are formed from a stale stage and
        // never used; for the first block of the walk, pprev and the V^T half
        // it meets are zero.
        qk_block<HD, QB>(lds + (KB == 0 ? ST : (ST + 1) % NS) * C::KBYTES, KB ^ 1, qop, snext, lane);
        if constexpr (KB == 0) {
          pv_block<HD, QB>(lds + vregion + SP * C::VBYTES, 1, pprev, o, lane);
        } else {
          pv_block<HD, QB>(vst, 0, pprev, o, lane);
        }
        float bsum[QB];
        softmax_block<QB>(scur, c2, mref, pprev, bsum);
        // Instruction order of the step: four LDS operand reads ahead, then
        // groups of (MFMA, one exp2, 2 other VALU, LDS read).  The VALU mask
        // (0x002) does not take transcendentals; they get their own groups
        // (0x400), one per MFMA.
        constexpr int kAhead = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
  #pragma unroll
        for (int i = 0; i < 16 - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
  #pragma unroll
        for (int i = 0; i < kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x400, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        settle(bsum, pprev, kst, KB, valid - 32 * KB);
      }
      if constexpr (KB == 0) {
        if (active && valid < 64) mask_block<QB>(snext, valid - 32, lane);
      } else {
        cur.next();
        if (has_next && active && cur.valid() < 32) mask_block<QB>(snext, cur.valid(), lane);
      }
    };
    auto tile = [&](int n, auto stage_tag) __attribute__((always_inline)) {
      step(n, stage_tag, std::integral_constant<int, 0>{}, sa, sb);
      step(n, stage_tag, std::integral_constant<int, 1>{}, sb, sa);
    };

    static_assert(NS == 4, "the tile loop below is unrolled for a 4-stage ring");
    for (int n = 0; n < total_tiles; n += NS) {
      tile(n, std::integral_constant<int, 0>{});
      if (n + 1 < total_tiles) tile(n + 1, std::integral_constant<int, 1>{});
      if (n + 2 < total_tiles) tile(n + 2, std::integral_constant<int, 2>{});
      if (n + 3 < total_tiles) tile(n + 3, std::integral_constant<int, 3>{});
    }
    // P.V of the last block (block 1 of the last tile).
    if (active) pv_block<HD, QB>(lds + vregion + ((total_tiles - 1) % NS) * C::VBYTES, 1, pprev, o, lane);

    __builtin_amdgcn_s_setprio(0);
    // Epilogue: O = O^T / l, LSE = ln2 * (mref + log2 l).
    if (!active) return;
    const int64_t orow_stride = (int64_t)a.heads * HD;
  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float ltot = halfwave_sum(l[qb]);
      const float inv = 1.0f / ltot;
      const float lse = (mref[qb] + __log2f(ltot)) * 0.69314718055994531f;
      const int r = (wv * QB + qb) * 32 + (lane & 31);
      if (r < q_rows) {
        const int64_t grow = q_offset + q_start + r;
        if (partial) {
          const int64_t prow = prow0 + r;
          float* orow = a.part_o + (((int64_t)split * a.part_rows + prow) * a.heads + h) * HD;
  #pragma unroll
          for (int db = 0; db < C::ND; ++db)
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              f32x4 v;
  #pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = o[db][qb][4 * g + i] * inv;
              *reinterpret_cast<f32x4*>(orow + db * 32 + g * 8 + (lane >> 5) * 4) = v;
            }
          if (lane < 32) a.part_lse[((int64_t)split * a.heads + h) * a.part_rows + prow] = lse;
        } else {
          __bf16* orow = static_cast<__bf16*>(a.o) + grow * orow_stride + (int64_t)h * HD;
          float sq = 0.0f;  // sum of squares of the row's bf16 outputs (this lane's half)
  #pragma unroll
          for (int db = 0; db < C::ND; ++db)
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              bf16x4 v;
  #pragma unroll
              for (int i = 0; i < 4; ++i) {
                v[i] = (__bf16)(o[db][qb][4 * g + i] * inv);
                sq = __builtin_fmaf((float)v[i], (float)v[i], sq);
              }
              *reinterpret_cast<bf16x4*>(orow + db * 32 + g * 8 + (lane >> 5) * 4) = v;
            }
          if (a.lse != nullptr && lane < 32) a.lse[(int64_t)h * a.lse_stride + grow] = lse;
          if (a.row_sq != nullptr) {
            // lanes l and l^32 hold the two halves of the row's dims (and
            // share r, so both take this branch)
            sq = halfwave_sum(sq);
            if (lane < 32) a.row_sq[grow * a.heads + h] = sq;
          }
        }
      }
    }
  };
  if (SPLIT || q_rows < kQTile) run(std::true_type{});
  else run(std::false_type{});
}

// Merge of partial results (one thread per partial row, head and 8 output
// dims): with per-split LSE s_k and normalised partial outputs O_k,
// LSE = log sum_k exp(s_k) and O = sum_k exp(s_k - LSE) O_k.  Splits with an
// empty key range carry s_k = -inf and weigh nothing.  TAIL: partial rows are
// the tail items' 256-row tiles, mapped to round rows through the work list
// (rows past an item's q_rows are skipped); otherwise they are round rows.
template <int HD, bool TAIL>
__global__ __launch_bounds__(256) void wave_attn_combine_kernel(AttnArgs a) {
  const int64_t prows = a.part_rows;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunks = HD / 8;
  if (t >= prows * a.heads * chunks) return;
  const int ch = (int)(t % chunks);
  const int64_t rh = t / chunks;
  const int h = (int)(rh % a.heads);
  const int64_t prow = rh / a.heads;
  int64_t row = prow;
  int S = a.num_splits;
  if constexpr (TAIL) {
    const int32_t* wk = a.work + 4 * (a.work_begin + a.num_direct + (int)(prow / kQTile));
    const int r = (int)(prow % kQTile);
    if (r >= wk[2]) return;
    row = (int64_t)a.nodes[kDescNodeWords * wk[0]] + wk[1] + r;
    S = a.tail_splits;
  }
  const int64_t rows = a.lse_stride;
  float smax = -INFINITY;
  for (int k = 0; k < S; ++k) smax = fmaxf(smax, a.part_lse[((int64_t)k * a.heads + h) * prows + prow]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float wsum = 0.0f;
  for (int k = 0; k < S; ++k) {
    const float sk = a.part_lse[((int64_t)k * a.heads + h) * prows + prow];
    if (sk == -INFINITY) continue;
    const float w = __expf(sk - smax);
    wsum += w;
    const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + (((int64_t)k * prows + prow) * a.heads + h) * HD + ch * 8);
    const f32x4 x = src[0], y = src[1];
    for (int i = 0; i < 4; ++i) {
      acc[i] += w * x[i];
      acc[4 + i] += w * y[i];
    }
  }
  const float inv = 1.0f / wsum;
  bf16x8 out;
  float sq = 0.0f;
  for (int i = 0; i < 8; ++i) {
    out[i] = (__bf16)(acc[i] * inv);
    sq = __builtin_fmaf((float)out[i], (float)out[i], sq);
  }
  *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.o) + (row * a.heads + h) * HD + ch * 8) = out;
  if (ch == 0 && a.lse != nullptr) a.lse[(int64_t)h * rows + row] = smax + __logf(wsum);
  if (a.row_sq != nullptr) {
    // The `chunks` threads of one (row, head) are consecutive and aligned in
    // the wave, and return early (above) all together or not at all.
    for (int m = chunks / 2; m >= 1; m >>= 1) sq += __shfl_xor(sq, m, chunks);
    if (ch == 0) a.row_sq[row * a.heads + h] = sq;
  }
}

template <bool TAIL>
hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.part_rows * a.heads * (a.head_dim / 8);
  dim3 cgrid((unsigned)((threads + 255) / 256));
  if (a.head_dim == 128) hipLaunchKernelGGL((wave_attn_combine_kernel<128, TAIL>), cgrid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((wave_attn_combine_kernel<64, TAIL>), cgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// 8 waves of 32 query rows: two waves per SIMD at 216 VGPRs.
constexpr int kWaves = 8;
constexpr int kQB = kQTile / (32 * kWaves);

}  // namespace

// Scratch of the allocation-free split-KV entry point: partial O and LSE of
// one call.  Each device holds its own copy for the life of the process; in
// host code `scratch` names a host-side stand-in, so kernels only ever get
// the device address that scratch_buffer() looks up.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // First call on this device (which is current here): look up this
    // device's copy of the array once and keep its address.
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_wave_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.num_work == 0) return hipSuccess;
  dim3 block(64 * kWaves);
  if (a.num_splits <= 1) {
    const int tail_items = a.num_work - a.num_direct;
    dim3 grid(a.num_direct * a.heads + tail_items * a.heads * a.tail_splits);
    if (a.head_dim == 128) hipLaunchKernelGGL((wave_attn_kernel<128, kWaves, kQB, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((wave_attn_kernel<64, kWaves, kQB, false>), grid, block, 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || tail_items == 0) return e;
    return launch_combine<true>(a, stream);
  }
  dim3 grid(a.num_work * a.heads * a.num_splits);
  if (a.head_dim == 128) hipLaunchKernelGGL((wave_attn_kernel<128, kWaves, kQB, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((wave_attn_kernel<64, kWaves, kQB, true>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine<false>(a, stream);
}

}  // namespace wave
