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
// head; 4 waves, one per SIMD, 64 query rows each.  Key tiles of 64 keys
// stream through a 3-stage LDS ring filled by direct global->LDS 16-byte
// loads.
//
// Contraction layout (bf16 MFMA 32x32x16, fp32 accumulation):
//   S^T[key][query] = K . Q^T   A = K rows from LDS, B = Q from registers.
//     With keys on the MFMA row axis, one lane holds one query and 16 keys,
//     so the softmax row max and row sum are in-lane except one exchange
//     between the two half-waves.  The K rows are stored permuted in LDS so
//     that a lane's 16 accumulator registers are 16 consecutive keys.
//   O^T[d][query] += V^T . P^T  A = V^T rows from LDS, B = P straight from the
//     softmax registers (bf16), no data movement.
// Online softmax in fp32 with exp2 and the scale folded into one FMA
// (FlashAttention-2 style deferred 1/l normalisation).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace wave {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKT = 64;     // keys per tile
constexpr int kStages = 3;  // LDS ring depth
constexpr int kMaxCtx = 512; // gather-list entries staged in LDS

template <int HD>
struct Cfg {
  static constexpr int KROW = HD * 2;     // bytes per K row in LDS
  static constexpr int KBYTES = kKT * KROW;
  static constexpr int VROW = kKT * 2;    // bytes per V^T row in LDS
  static constexpr int VBYTES = HD * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NC = HD / 16;      // k-steps of Q.K^T
  static constexpr int ND = HD / 32;      // d blocks of O^T
  static constexpr int KLOADS = KBYTES / (kThreads * 16);
  static constexpr int VLOADS = VBYTES / (kThreads * 16);
  static constexpr int LOADS = KLOADS + VLOADS;
};

// 16-byte chunk swizzles inside an LDS row: an MFMA operand read has 8 (16)
// consecutive lanes on consecutive rows and the same logical chunk; these
// put them on distinct banks for 128-byte and 256-byte bank windows.
__device__ __forceinline__ int swz16(int row) { return row & 15; }               // 256-byte rows
__device__ __forceinline__ int swz8(int row) { return (row + (row >> 3)) & 7; }  // 128-byte rows

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

typedef __attribute__((address_space(3))) void lds_void;

template <int HD>
__device__ __forceinline__ void issue_tile(char* stage, const __bf16* kslot, const __bf16* vtslot,
                                           int key0, int lpad, int wv, int lane) {
  using C = Cfg<HD>;
#pragma unroll
  for (int n = 0; n < C::KLOADS; ++n) {
    const int chunk_base = (wv * C::KLOADS + n) * 1024;
    const int off = chunk_base + lane * 16;
    const int row = off / C::KROW;
    const int pc = (off % C::KROW) / 16;
    const int lc = pc ^ swzK<HD>(row);
    const __bf16* g = kslot + (int64_t)(key0 + perm_key(row)) * HD + lc * 8;
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(stage + chunk_base), 16, 0, 0);
  }
#pragma unroll
  for (int n = 0; n < C::VLOADS; ++n) {
    const int chunk_base = (wv * C::VLOADS + n) * 1024;
    const int off = chunk_base + lane * 16;
    const int d = off / C::VROW;
    const int pc = (off % C::VROW) / 16;
    const int lc = pc ^ swz8(d);
    const __bf16* g = vtslot + (int64_t)d * lpad + key0 + lc * 8;
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(stage + C::KBYTES + chunk_base), 16, 0, 0);
  }
}

template <int HD>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void wave_attn_kernel(AttnArgs a) {
  using C = Cfg<HD>;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * C::STAGE];
  __shared__ int ctx_lds[2 * kMaxCtx];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int item = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
  const int32_t* wk = a.work + 4 * (a.work_begin + item);
  const int node = wk[0], q_start = wk[1], q_rows = wk[2];
  const int32_t* nd = a.nodes + 4 * node;
  const int q_offset = nd[0], ctx_count = nd[3];
  const int32_t* ctx_g = a.ctx + 2 * nd[2];
  const int lpad = a.lpad;
  const int64_t slot_elems = (int64_t)a.heads * lpad * HD;
  const __bf16* kcache = static_cast<const __bf16*>(a.k) + (int64_t)h * lpad * HD;
  const __bf16* vcache = static_cast<const __bf16*>(a.vt) + (int64_t)h * HD * lpad;

  // The gather list goes to LDS once, so that walking it inside the tile
  // loop never waits on the vector-memory counter the K/V prefetch uses.
  for (int e = threadIdx.x; e < 2 * ctx_count; e += kThreads) ctx_lds[e] = ctx_g[e];
  __syncthreads();
  const int* ctx = ctx_lds;
  int total_tiles = 0;
  for (int e = 0; e < ctx_count; ++e) total_tiles += (ctx[2 * e + 1] + kKT - 1) / kKT;

  // Q fragments (B operand of S^T): lane holds query (lane & 31) of block qb,
  // dims 16c + 8*(lane>>5) .. +7.
  bf16x8 qop[2][C::NC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = wv * 64 + qb * 32 + (lane & 31);
    const bool valid = r < q_rows;
    const int64_t base = (int64_t)(q_offset + q_start + r) * a.q_row_stride + (int64_t)h * HD + 8 * (lane >> 5);
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      bf16x8 v;
      if (!valid) {
        for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
      } else if (a.q_fp32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.q) + base + 16 * c);
        const f32x4 x = p[0], y = p[1];
        v[0] = (__bf16)x[0]; v[1] = (__bf16)x[1]; v[2] = (__bf16)x[2]; v[3] = (__bf16)x[3];
        v[4] = (__bf16)y[0]; v[5] = (__bf16)y[1]; v[6] = (__bf16)y[2]; v[7] = (__bf16)y[3];
      } else {
        v = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + base + 16 * c);
      }
      qop[qb][c] = v;
    }
  }

  f32x16 o[C::ND][2];
#pragma unroll
  for (int db = 0; db < C::ND; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.0f;
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.0f, 0.0f};
  const float c2 = a.scale_log2e;

  // Load iterator.
  int le = 0, lt = 0;
  auto next_load = [&](int stage) {
    const int phys = ctx[2 * le];
    const int len = ctx[2 * le + 1];
    issue_tile<HD>(lds + stage * C::STAGE, kcache + phys * slot_elems, vcache + phys * slot_elems,
                   lt * kKT, lpad, wv, lane);
    if ((lt + 1) * kKT >= len) {
      ++le;
      lt = 0;
    } else {
      ++lt;
    }
  };
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < total_tiles) next_load(s);

  int ce = 0, ct = 0;  // compute iterator
  for (int n = 0; n < total_tiles; ++n) {
    if (n + 1 < total_tiles) {
      // tile n+1 may still be in flight
      __builtin_amdgcn_s_waitcnt((C::LOADS & 15) | ((C::LOADS >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    }
    // Raw barrier: the counters above already cover this thread's LDS fills,
    // and every wave finished reading the stage about to be refilled.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (n + kStages - 1 < total_tiles) next_load((n + kStages - 1) % kStages);

    const char* ks = lds + (n % kStages) * C::STAGE;
    const char* vs = ks + C::KBYTES;
    const int len = ctx[2 * ce + 1];
    const int key0 = ct * kKT;

    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 32 + (lane & 31);
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        const int ch = 2 * c + (lane >> 5);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(ks + row * C::KROW + ((ch ^ swzK<HD>(row)) * 16));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qop[qb][c], s[kb][qb], 0, 0, 0);
      }
    }
    if (key0 + kKT > len) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + kb * 32 + (lane >> 5) * 16 + r >= len) s[kb][qb][r] = -INFINITY;
    }

    bf16x8 pop[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[qb] - mnew) * c2);
      m[qb] = mnew;
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
      const float nm = -mnew * c2;
      float sum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 pv;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * hh + t], c2, nm));
            sum += p;
            pv[t] = (__bf16)p;
          }
          pop[kb][qb][hh] = pv;
        }
      l[qb] += sum;
    }

#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
      const int d = db * 32 + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kc = 4 * kb + 2 * (lane >> 5) + hh;
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vs + d * C::VROW + ((kc ^ swz8(d)) * 16));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pop[kb][qb][hh], o[db][qb], 0, 0, 0);
        }
    }

    if ((ct + 1) * kKT >= len) {
      ++ce;
      ct = 0;
    } else {
      ++ct;
    }
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m * c2 + log2 l).
  __bf16* out = static_cast<__bf16*>(a.o);
  const int64_t orow_stride = (int64_t)a.heads * HD;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = 1.0f / ltot;
    const int r = wv * 64 + qb * 32 + (lane & 31);
    if (r < q_rows) {
      const int64_t grow = q_offset + q_start + r;
      __bf16* orow = out + grow * orow_stride + (int64_t)h * HD;
#pragma unroll
      for (int db = 0; db < C::ND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (__bf16)(o[db][qb][4 * g + i] * inv);
          *reinterpret_cast<bf16x4*>(orow + db * 32 + g * 8 + (lane >> 5) * 4) = v;
        }
      if (a.lse != nullptr && lane < 32)
        a.lse[(int64_t)h * a.lse_stride + grow] = (m[qb] * c2 + __log2f(ltot)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

hipError_t launch_wave_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.num_work == 0) return hipSuccess;
  dim3 grid(a.num_work * a.heads);
  dim3 block(kThreads);
  if (a.head_dim == 128) hipLaunchKernelGGL((wave_attn_kernel<128>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((wave_attn_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace wave
