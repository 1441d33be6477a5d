// kv_write: copy one round's fresh K/V into physical cache slots (gfx950).
//
// The runtime writes each chunk's fresh K/V into a cache as soon as it is
// produced, so later chunks of the same round can read it (Wave Forcing
// summary on aiany.app, mechanism paragraph: early K/V delivery; Wan-Streamer
// v0.2 abstract: incoming K/V written into a local cache).
//
// Source rows are token-major [token][head][d] (the layout a QKV projection
// emits).  The cache keeps, per slot and head, K token-major [lpad][d] and V
// transposed [d][lpad]; tokens [len, lpad) are zeroed so that a full key tile
// read past the slot's end multiplies zeros.  fp32 sources are rounded to
// bf16 to nearest even.  Pure data movement: HBM-bound.  With stream_out the
// cache stores are non-temporal (decode-shaped rounds; see abi.cpp).
//
// Grid: (lpad / 64 token tiles, writes, heads); 256 threads; one block moves
// 64 tokens x d of one head of one slot.  V goes through LDS for the
// transpose; every global access is a 16-byte vector.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.hpp"

namespace wave {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;
constexpr int kThreads = 256;

template <bool FP32>
__device__ inline bf16x8 load8(const void* base, int64_t elem) {
  if constexpr (FP32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + elem);
    const f32x4 a = p[0], b = p[1];
    bf16x8 r;
    r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
    r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
    return r;
  } else {
    return *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(base) + elem);
  }
}

template <bool NT>
__device__ inline void store16(__bf16* dst, bf16x8 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(dst));
  else *reinterpret_cast<bf16x8*>(dst) = v;
}

template <int HD, bool FP32, bool NT>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteArgs a) {
  constexpr int CH = HD / 8;        // 16-byte chunks per token row
  constexpr int LDS_STRIDE = HD + 8; // bf16 elements per staged row (pad against conflicts)
  __shared__ __attribute__((aligned(16))) __bf16 vtile[kTok * LDS_STRIDE];

  const int tile = blockIdx.x, w = blockIdx.y, h = blockIdx.z;
  const int32_t* wr = a.writes + 4 * w;
  const int slot = wr[0], len = wr[1], src_off = wr[2];
  const int tok0 = tile * kTok;
  const int64_t kbase = ((int64_t)slot * a.heads + h) * a.lpad * HD;
  const int64_t vbase = ((int64_t)slot * a.heads + h) * HD * (int64_t)a.lpad;
  __bf16* kc = static_cast<__bf16*>(a.k);
  __bf16* vt = static_cast<__bf16*>(a.vt);

  // K rows and the V tile into LDS.
  for (int c = threadIdx.x; c < kTok * CH; c += kThreads) {
    const int row = c / CH, ch = c % CH;
    const int tok = tok0 + row;
    bf16x8 kv, vv;
    if (tok < len) {
      const int64_t e = (int64_t)(src_off + tok) * a.src_row_stride + (int64_t)h * HD + ch * 8;
      kv = load8<FP32>(a.k_src, e);
      vv = load8<FP32>(a.v_src, e);
    } else {
      for (int i = 0; i < 8; ++i) { kv[i] = (__bf16)0.0f; vv[i] = (__bf16)0.0f; }
    }
    store16<NT>(kc + kbase + (int64_t)tok * HD + ch * 8, kv);
    *reinterpret_cast<bf16x8*>(&vtile[row * LDS_STRIDE + ch * 8]) = vv;
  }
  __syncthreads();
  // V^T rows: d-major, 64 tokens = 8 chunks of 8 per row.
  for (int c = threadIdx.x; c < HD * (kTok / 8); c += kThreads) {
    const int d = c / (kTok / 8), tc = c % (kTok / 8);
    bf16x8 out;
    for (int i = 0; i < 8; ++i) out[i] = vtile[(tc * 8 + i) * LDS_STRIDE + d];
    store16<NT>(vt + vbase + (int64_t)d * a.lpad + tok0 + tc * 8, out);
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  if (a.num_writes == 0) return hipSuccess;
  dim3 grid(a.lpad / kTok, a.num_writes, a.heads);
  dim3 block(kThreads);
  auto go = [&](auto hd, auto fp32) {
    constexpr int H = decltype(hd)::value;
    constexpr bool F = decltype(fp32)::value;
    if (a.stream_out) hipLaunchKernelGGL((kv_write_kernel<H, F, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((kv_write_kernel<H, F, false>), grid, block, 0, stream, a);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  if (a.head_dim == 128) {
    if (a.src_fp32) go(I128{}, std::true_type{});
    else go(I128{}, std::false_type{});
  } else {
    if (a.src_fp32) go(I64{}, std::true_type{});
    else go(I64{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace wave
