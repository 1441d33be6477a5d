// C ABI shim: argument validation, error reporting and kernel launches.
// No C++ exception crosses this boundary; every entry point returns a status.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "balance.hpp"
#include "kernels.hpp"
#include "planner.hpp"
#include "wave.h"

static_assert(wave::kNodeStride == wave::kDescNodeWords, "descriptor node rows: planner and kernels disagree");

struct wave_plan {
  wave::Plan p;
  // tail-balancing choices, memoised per (round, heads, head_dim, compute units)
  mutable std::mutex mu;
  mutable std::map<std::array<int32_t, 4>, wave::TailSplit> tails;
};

namespace {

thread_local std::string g_last_error;

int32_t set_error(int32_t code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return WAVE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by kv_write and wave_attn.
int32_t check_common(const wave_plan_t* plan, const void* d_desc, int32_t round,
                     const wave_kv_cache* cache, const char* fn) {
  const std::string f(fn);
  if (!plan || !d_desc || !cache) return set_error(WAVE_ERR_INVALID_ARG, f + ": null plan, descriptor or cache");
  const wave::Plan& p = plan->p;
  if (round < 0 || round >= p.num_rounds())
    return set_error(WAVE_ERR_INVALID_ARG, f + ": round out of range");
  if (!cache->k || !cache->vt) return set_error(WAVE_ERR_INVALID_ARG, f + ": null cache buffer");
  if (!aligned16(cache->k) || !aligned16(cache->vt) || !aligned16(d_desc))
    return set_error(WAVE_ERR_INVALID_ARG, f + ": cache buffers and descriptor must be 16-byte aligned");
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
  if (cache->heads < 1 || cache->heads > 65535) return set_error(WAVE_ERR_INVALID_ARG, f + ": heads out of range");
  if (cache->lpad < 1 || cache->lpad % WAVE_KEY_TILE != 0)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": lpad must be a positive multiple of WAVE_KEY_TILE");
  // The attention kernel addresses a lane's share of a V^T tile with a 32-bit
  // byte offset from the tile's first key: up to ((head_dim-1)*lpad + 56)*2
  // plus the 16 bytes it loads.
  if (static_cast<int64_t>(cache->head_dim - 1) * cache->lpad * 2 + 2 * WAVE_KEY_TILE > INT32_MAX)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": lpad too long for 32-bit V^T tile offsets");
  if (cache->lpad < p.max_slot_len)
    return set_error(WAVE_ERR_CAPACITY, f + ": lpad shorter than the plan's longest slot");
  if (cache->num_slots < p.num_phys_slots)
    return set_error(WAVE_ERR_CAPACITY, f + ": cache has fewer slots than the plan needs");
  return WAVE_OK;
}

// Validates kv_write's arguments and fills its launch arguments (num_writes
// = 0 for a round without writes, which launches nothing).
int32_t kv_prepare(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                   const void* k_src, const void* v_src, int32_t src_dtype, int64_t src_row_stride, const char* fn,
                   wave::KvWriteArgs& a) {
  int32_t rc = check_common(plan, d_desc, round, cache, fn);
  if (rc != WAVE_OK) return rc;
  const std::string f(fn);
  const wave::Plan& p = plan->p;
  const int32_t w0 = p.round_write_begin[round], w1 = p.round_write_begin[round + 1];
  a = wave::KvWriteArgs{};
  if (w1 == w0) return WAVE_OK;
  if (!k_src || !v_src) return set_error(WAVE_ERR_INVALID_ARG, f + ": null source");
  if (src_dtype != WAVE_DTYPE_BF16 && src_dtype != WAVE_DTYPE_FP32)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": src_dtype must be WAVE_DTYPE_BF16 or WAVE_DTYPE_FP32");
  const int64_t row = static_cast<int64_t>(cache->heads) * cache->head_dim;
  if (src_row_stride < row) return set_error(WAVE_ERR_INVALID_ARG, f + ": src_row_stride < heads*head_dim");
  const int64_t esz = src_dtype == WAVE_DTYPE_FP32 ? 4 : 2;
  if (!aligned16(k_src) || !aligned16(v_src) || (src_row_stride * esz) % 16 != 0)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": sources and row stride must be 16-byte aligned");
  const int32_t* desc = static_cast<const int32_t*>(d_desc);
  a.writes = desc + p.desc[10] + static_cast<int64_t>(w0) * wave::kWriteStride;
  a.num_writes = w1 - w0;
  a.k = cache->k;
  a.vt = cache->vt;
  a.heads = cache->heads;
  a.head_dim = cache->head_dim;
  a.lpad = cache->lpad;
  a.k_src = k_src;
  a.v_src = v_src;
  a.src_fp32 = src_dtype == WAVE_DTYPE_FP32;
  a.src_row_stride = src_row_stride;
  // Decode-shaped plans (queries shorter than the chunk): the round's
  // attention streams the whole history from HBM, so the fresh K/V go out
  // with non-temporal stores instead of sitting dirty in the last-level
  // cache, whose write-back would then compete with those reads.
  a.stream_out = p.params.query_len > 0 && p.params.query_len < p.params.chunk_len;
  return WAVE_OK;
}

}  // namespace

extern "C" {

int32_t wave_plan(const wave_plan_params* params, wave_plan_t** out) {
  if (!params || !out) return set_error(WAVE_ERR_INVALID_ARG, "wave_plan: null argument");
  *out = nullptr;
  try {
    wave_plan_t* h = new wave_plan_t();
    std::string err;
    const int32_t rc = wave::build_plan(*params, h->p, &err);
    if (rc != WAVE_OK) {
      delete h;
      return set_error(rc, err);
    }
    *out = h;
    return ok();
  } catch (const std::bad_alloc&) {
    return set_error(WAVE_ERR_NOMEM, "wave_plan: out of host memory");
  } catch (...) {
    return set_error(WAVE_ERR_INVALID_ARG, "wave_plan: unexpected failure");
  }
}

int32_t wave_plan_view_get(const wave_plan_t* plan, wave_plan_view* out) {
  if (!plan || !out) return set_error(WAVE_ERR_INVALID_ARG, "wave_plan_view_get: null argument");
  const wave::Plan& p = plan->p;
  out->num_rounds = p.num_rounds();
  out->num_nodes = static_cast<int32_t>(p.nodes.size());
  out->num_ctx = static_cast<int32_t>(p.ctx.size());
  out->num_writes = static_cast<int32_t>(p.writes.size());
  out->num_work = static_cast<int32_t>(p.work.size());
  out->num_phys_slots = p.num_phys_slots;
  out->max_slot_len = p.max_slot_len;
  out->q_tile = p.params.q_tile;
  out->round_node_begin = p.round_node_begin.data();
  out->round_write_begin = p.round_write_begin.data();
  out->round_work_begin = p.round_work_begin.data();
  out->round_q_rows = p.round_q_rows.data();
  out->round_src_rows = p.round_src_rows.data();
  out->nodes = p.nodes.data();
  out->ctx = p.ctx.data();
  out->writes = p.writes.data();
  out->work = p.work.data();
  return ok();
}

int32_t wave_plan_desc_size(const wave_plan_t* plan, size_t* bytes) {
  if (!plan || !bytes) return set_error(WAVE_ERR_INVALID_ARG, "wave_plan_desc_size: null argument");
  *bytes = plan->p.desc.size() * sizeof(int32_t);
  return ok();
}

int32_t wave_plan_desc_pack(const wave_plan_t* plan, void* host_dst, size_t bytes) {
  if (!plan || !host_dst) return set_error(WAVE_ERR_INVALID_ARG, "wave_plan_desc_pack: null argument");
  const size_t need = plan->p.desc.size() * sizeof(int32_t);
  if (bytes < need) return set_error(WAVE_ERR_INVALID_ARG, "wave_plan_desc_pack: destination too small");
  std::memcpy(host_dst, plan->p.desc.data(), need);
  return ok();
}

void wave_plan_destroy(wave_plan_t* plan) { delete plan; }

int32_t kv_write(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                 const void* k_src, const void* v_src, int32_t src_dtype, int64_t src_row_stride,
                 void* stream) {
  wave::KvWriteArgs a{};
  const int32_t rc = kv_prepare(plan, d_desc, round, cache, k_src, v_src, src_dtype, src_row_stride, "kv_write", a);
  if (rc != WAVE_OK) return rc;
  const hipError_t e = wave::launch_kv_write(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, std::string("kv_write: ") + hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Compute units of the current device (256 if it cannot be queried).
int32_t device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

// Splits for split-KV attention: the most whose workgroups fit the current
// device's compute units in one dispatch wave, 1..64.
int32_t auto_splits(const wave::Plan& p, int32_t round, int32_t heads, int32_t head_dim) {
  return wave::choose_splits(p, round, heads, head_dim, device_cus());
}

constexpr size_t kAlign = 256;

wave::TailSplit tail_for(const wave_plan_t* plan, int32_t round, int32_t heads, int32_t head_dim, int32_t cus) {
  const std::array<int32_t, 4> key{round, heads, head_dim, cus};
  std::lock_guard<std::mutex> lock(plan->mu);
  auto it = plan->tails.find(key);
  if (it != plan->tails.end()) return it->second;
  const wave::TailSplit t = wave::choose_tail_split(plan->p, round, heads, head_dim, cus);
  plan->tails.emplace(key, t);
  return t;
}

// Workspace of tail balancing: fp32 O [splits][items*256][heads][d], then
// (256-byte aligned) fp32 LSE [splits][heads][items*256].
size_t tail_bytes(const wave::TailSplit& t, int32_t heads, int32_t head_dim, size_t* lse_offset) {
  if (t.items == 0) {
    if (lse_offset) *lse_offset = 0;
    return 0;
  }
  const size_t prows = static_cast<size_t>(t.items) * WAVE_Q_TILE;
  const size_t o_bytes = static_cast<size_t>(t.splits) * prows * heads * head_dim * sizeof(float);
  const size_t off = (o_bytes + kAlign - 1) / kAlign * kAlign;
  if (lse_offset) *lse_offset = off;
  return off + static_cast<size_t>(t.splits) * heads * prows * sizeof(float);
}

size_t splitkv_bytes(const wave::Plan& p, int32_t round, int32_t heads, int32_t head_dim, int32_t splits,
                     size_t* lse_offset) {
  const size_t rows = static_cast<size_t>(p.round_q_rows[round]);
  const size_t o_bytes = static_cast<size_t>(splits) * rows * heads * head_dim * sizeof(float);
  const size_t off = (o_bytes + kAlign - 1) / kAlign * kAlign;
  if (lse_offset) *lse_offset = off;
  return off + static_cast<size_t>(splits) * heads * rows * sizeof(float);
}

int32_t attn_common(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                    const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                    const char* fn, wave::AttnArgs& a) {
  int32_t rc = check_common(plan, d_desc, round, cache, fn);
  if (rc != WAVE_OK) return rc;
  const std::string f(fn);
  const wave::Plan& p = plan->p;
  if (!q || !o) return set_error(WAVE_ERR_INVALID_ARG, f + ": null q or o");
  if (p.params.q_tile != WAVE_Q_TILE)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": plan q_tile must be WAVE_Q_TILE");
  if (p.max_ctx > 512) return set_error(WAVE_ERR_UNSUPPORTED, f + ": gather lists longer than 512 slots");
  if (q_dtype != WAVE_DTYPE_BF16 && q_dtype != WAVE_DTYPE_FP32)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": q_dtype must be WAVE_DTYPE_BF16 or WAVE_DTYPE_FP32");
  const int64_t row = static_cast<int64_t>(cache->heads) * cache->head_dim;
  if (q_row_stride < row) return set_error(WAVE_ERR_INVALID_ARG, f + ": q_row_stride < heads*head_dim");
  const int64_t esz = q_dtype == WAVE_DTYPE_FP32 ? 4 : 2;
  if (!aligned16(q) || (q_row_stride * esz) % 16 != 0 || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": q, o and q's rows must be 16-byte aligned, lse 4-byte");
  if (!std::isfinite(scale)) return set_error(WAVE_ERR_INVALID_ARG, f + ": scale must be finite");
  const int32_t k0 = p.round_work_begin[round], k1 = p.round_work_begin[round + 1];
  if (static_cast<int64_t>(k1 - k0) * cache->heads * 64 > INT32_MAX)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": too many work items");
  const int32_t* desc = static_cast<const int32_t*>(d_desc);
  a = wave::AttnArgs{};
  a.nodes = desc + p.desc[8];
  a.ctx = desc + p.desc[9];
  a.work = desc + p.desc[11];
  a.work_begin = k0;
  a.num_work = k1 - k0;
  a.k = cache->k;
  a.vt = cache->vt;
  a.heads = cache->heads;
  a.head_dim = cache->head_dim;
  a.lpad = cache->lpad;
  a.q = q;
  a.q_fp32 = q_dtype == WAVE_DTYPE_FP32;
  a.q_row_stride = q_row_stride;
  a.o = o;
  a.lse = lse;
  a.lse_stride = p.round_q_rows[round];
  a.scale_log2e = scale * 1.4426950408889634f;
  a.num_splits = 1;
  a.num_direct = a.num_work;
  a.tail_splits = 1;
  a.part_rows = 0;
  return WAVE_OK;
}

// wave_attn's checks plus its optional tail-balancing workspace.
int32_t attn_prepare(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                     const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                     void* workspace, size_t workspace_bytes, const char* fn, wave::AttnArgs& a) {
  const int32_t rc = attn_common(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale, fn, a);
  if (rc != WAVE_OK) return rc;
  if (!workspace) return WAVE_OK;
  const std::string f(fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": workspace must be 256-byte aligned");
  const wave::TailSplit t = tail_for(plan, round, cache->heads, cache->head_dim, device_cus());
  size_t lse_off = 0;
  const size_t need = tail_bytes(t, cache->heads, cache->head_dim, &lse_off);
  if (workspace_bytes < need)
    return set_error(WAVE_ERR_CAPACITY, f + ": workspace smaller than wave_attn_workspace()");
  if (t.items > 0) {
    if (static_cast<int64_t>(a.num_work) * cache->heads * t.splits > INT32_MAX)
      return set_error(WAVE_ERR_UNSUPPORTED, f + ": too many workgroups");
    a.num_direct = a.num_work - t.items;
    a.tail_splits = t.splits;
    a.part_rows = t.items * WAVE_Q_TILE;
    a.part_o = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off);
  }
  return WAVE_OK;
}

}  // namespace

extern "C" {

int32_t wave_attn_workspace(const wave_plan_t* plan, int32_t round, int32_t heads, int32_t head_dim,
                            int32_t compute_units, size_t* bytes, int32_t* tail_items, int32_t* tail_splits) {
  if (!plan || !bytes) return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_workspace: null argument");
  const wave::Plan& p = plan->p;
  if (round < 0 || round >= p.num_rounds())
    return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_workspace: round out of range");
  if (heads < 1 || heads > 65535 || (head_dim != 64 && head_dim != 128) || compute_units < 0)
    return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_workspace: bad heads, head_dim or compute_units");
  const wave::TailSplit t =
      tail_for(plan, round, heads, head_dim, compute_units == 0 ? device_cus() : compute_units);
  *bytes = tail_bytes(t, heads, head_dim, nullptr);
  if (tail_items) *tail_items = t.items;
  if (tail_splits) *tail_splits = t.splits;
  return ok();
}

int32_t wave_attn(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                  const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                  void* workspace, size_t workspace_bytes, void* stream) {
  wave::AttnArgs a;
  const int32_t rc = attn_prepare(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale, workspace,
                                  workspace_bytes, "wave_attn", a);
  if (rc != WAVE_OK) return rc;
  const hipError_t e = wave::launch_wave_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, std::string("wave_attn: ") + hipGetErrorString(e));
  return ok();
}

int32_t wave_attn_chain(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                        const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                        float* row_sq, void* workspace, size_t workspace_bytes, void* stream) {
  wave::AttnArgs a;
  const int32_t rc = attn_prepare(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale, workspace,
                                  workspace_bytes, "wave_attn_chain", a);
  if (rc != WAVE_OK) return rc;
  if (row_sq && (reinterpret_cast<uintptr_t>(row_sq) & 3u) != 0)
    return set_error(WAVE_ERR_UNSUPPORTED, "wave_attn_chain: row_sq must be 4-byte aligned");
  a.row_sq = row_sq;
  const hipError_t e = wave::launch_wave_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, std::string("wave_attn_chain: ") + hipGetErrorString(e));
  return ok();
}

int32_t wave_round(const wave_plan_t* plan, const void* d_desc, int32_t round, int32_t num_layers,
                   const wave_kv_cache* caches, const void* const* k_src, const void* const* v_src, int32_t src_dtype,
                   int64_t src_row_stride, const void* const* q, int32_t q_dtype, int64_t q_row_stride,
                   void* const* o, float* const* lse, float scale, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (num_layers < 1 || !caches || !k_src || !v_src || !q || !o)
    return set_error(WAVE_ERR_INVALID_ARG, "wave_round: num_layers < 1 or a null per-layer array");
  try {
    // Every layer's arguments are checked before anything is enqueued.
    std::vector<wave::KvWriteArgs> kw(static_cast<size_t>(num_layers));
    std::vector<wave::AttnArgs> at(static_cast<size_t>(num_layers));
    for (int32_t l = 0; l < num_layers; ++l) {
      const std::string fn = "wave_round (layer " + std::to_string(l) + ")";
      int32_t rc = kv_prepare(plan, d_desc, round, &caches[l], k_src[l], v_src[l], src_dtype, src_row_stride,
                              fn.c_str(), kw[l]);
      if (rc != WAVE_OK) return rc;
      rc = attn_prepare(plan, d_desc, round, &caches[l], q[l], q_dtype, q_row_stride, o[l], lse ? lse[l] : nullptr,
                        scale, workspace, workspace_bytes, fn.c_str(), at[l]);
      if (rc != WAVE_OK) return rc;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t l = 0; l < num_layers; ++l) {
      hipError_t e = wave::launch_kv_write(kw[l], st);
      if (e == hipSuccess) e = wave::launch_wave_attn(at[l], st);
      if (e != hipSuccess)
        return set_error(WAVE_ERR_HIP, "wave_round (layer " + std::to_string(l) + "): " + hipGetErrorString(e));
    }
    return ok();
  } catch (const std::bad_alloc&) {
    return set_error(WAVE_ERR_NOMEM, "wave_round: out of host memory");
  }
}

int32_t wave_attn_splitkv_workspace(const wave_plan_t* plan, int32_t round, int32_t heads, int32_t head_dim,
                                    int32_t num_splits, size_t* bytes, int32_t* splits_used) {
  if (!plan || !bytes) return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_splitkv_workspace: null argument");
  const wave::Plan& p = plan->p;
  if (round < 0 || round >= p.num_rounds())
    return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_splitkv_workspace: round out of range");
  if (heads < 1 || head_dim < 1 || num_splits < 0 || num_splits > 4096)
    return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_splitkv_workspace: bad heads, head_dim or num_splits");
  const int32_t s = num_splits == 0 ? auto_splits(p, round, heads, head_dim) : num_splits;
  *bytes = splitkv_bytes(p, round, heads, head_dim, s, nullptr);
  if (splits_used) *splits_used = s;
  return ok();
}

}  // extern "C"

namespace {

// Checks of the split-KV calls; fills the launch arguments except the
// partial-result pointers and returns the workspace the call needs.
int32_t splitkv_prepare(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                        const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                        int32_t num_splits, const char* fn, wave::AttnArgs& a, size_t* need, size_t* lse_off) {
  const int32_t rc = attn_common(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale, fn, a);
  if (rc != WAVE_OK) return rc;
  const std::string f(fn);
  if (num_splits < 0 || num_splits > 4096)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": num_splits must be in [0, 4096]");
  const wave::Plan& p = plan->p;
  const int32_t s = num_splits == 0 ? auto_splits(p, round, cache->heads, cache->head_dim) : num_splits;
  if (static_cast<int64_t>(a.num_work) * cache->heads * s > INT32_MAX)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": too many workgroups");
  *need = splitkv_bytes(p, round, cache->heads, cache->head_dim, s, lse_off);
  a.num_splits = s;
  a.part_rows = p.round_q_rows[round];
  return WAVE_OK;
}

int32_t splitkv_launch(wave::AttnArgs& a, void* scratch, size_t lse_off, void* stream, const char* fn) {
  if (a.num_splits > 1) {
    a.part_o = static_cast<float*>(scratch);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(scratch) + lse_off);
  } else {
    // one split: the plain kernel writes o and lse directly
    a.part_o = nullptr;
    a.part_lse = nullptr;
  }
  const hipError_t e = wave::launch_wave_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, std::string(fn) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t wave_attn_splitkv(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                          const void* q, int32_t q_dtype, int64_t q_row_stride, void* o, float* lse, float scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  wave::AttnArgs a;
  size_t need = 0, lse_off = 0;
  const char* fn = "wave_attn_splitkv";
  const int32_t rc = splitkv_prepare(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale,
                                     num_splits, fn, a, &need, &lse_off);
  if (rc != WAVE_OK) return rc;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return set_error(WAVE_ERR_INVALID_ARG, "wave_attn_splitkv: workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < need)
    return set_error(WAVE_ERR_CAPACITY, "wave_attn_splitkv: workspace smaller than wave_attn_splitkv_workspace()");
  return splitkv_launch(a, workspace, lse_off, stream, fn);
}

int32_t wave_attn_splitkv_noalloc(const wave_plan_t* plan, const void* d_desc, int32_t round,
                                  const wave_kv_cache* cache, const void* q, int32_t q_dtype, int64_t q_row_stride,
                                  void* o, float* lse, float scale, int32_t num_splits, void* stream) {
  static_assert(wave::kScratchBytes == WAVE_NOALLOC_SCRATCH_BYTES, "scratch size: header and library disagree");
  wave::AttnArgs a;
  size_t need = 0, lse_off = 0;
  const char* fn = "wave_attn_splitkv_noalloc";
  const int32_t rc = splitkv_prepare(plan, d_desc, round, cache, q, q_dtype, q_row_stride, o, lse, scale,
                                     num_splits, fn, a, &need, &lse_off);
  if (rc != WAVE_OK) return rc;
  void* scratch = nullptr;
  if (a.num_splits > 1) {
    if (need > wave::kScratchBytes)
      return set_error(WAVE_ERR_CAPACITY, std::string(fn) + ": the call needs " + std::to_string(need) +
                                              " bytes of scratch, above WAVE_NOALLOC_SCRATCH_BYTES (" +
                                              std::to_string(wave::kScratchBytes) +
                                              "); use fewer splits, or wave_attn_splitkv with a workspace");
    const hipError_t e = wave::scratch_buffer(&scratch);
    if (e != hipSuccess) return set_error(WAVE_ERR_HIP, std::string(fn) + ": scratch lookup: " + hipGetErrorString(e));
  }
  return splitkv_launch(a, scratch, lse_off, stream, fn);
}

}  // extern "C"

namespace {

int32_t chain_plan_check(const wave::Plan& p, const std::string& f) {
  if (p.params.cond_len != 0 || (p.params.query_len != 0 && p.params.query_len != p.params.chunk_len))
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": the chain needs cond_len = 0 and query rows = chunk tokens");
  return WAVE_OK;
}

}  // namespace

extern "C" {

int32_t qkv_project_workspace(const wave_plan_t* plan, int32_t round, size_t* bytes) {
  if (!plan || !bytes) return set_error(WAVE_ERR_INVALID_ARG, "qkv_project_workspace: null argument");
  const wave::Plan& p = plan->p;
  if (round < 0 || round >= p.num_rounds())
    return set_error(WAVE_ERR_INVALID_ARG, "qkv_project_workspace: round out of range");
  *bytes = static_cast<size_t>(p.round_q_rows[round]) * sizeof(float);
  return ok();
}

int32_t qkv_project(const wave_plan_t* plan, const void* d_desc, int32_t round, const wave_kv_cache* cache,
                    const void* x, int32_t x_layout, const float* row_sq, const void* w, void* q, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const std::string f("qkv_project");
  int32_t rc = check_common(plan, d_desc, round, cache, "qkv_project");
  if (rc != WAVE_OK) return rc;
  const wave::Plan& p = plan->p;
  rc = chain_plan_check(p, f);
  if (rc != WAVE_OK) return rc;
  if (!x || !w || !q) return set_error(WAVE_ERR_INVALID_ARG, f + ": null x, w or q");
  if (x_layout != WAVE_X_ROUND && x_layout != WAVE_X_CHUNK)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": x_layout must be WAVE_X_ROUND or WAVE_X_CHUNK");
  if (!aligned16(x) || !aligned16(w) || !aligned16(q))
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": x, w and q must be 16-byte aligned");
  if (row_sq && x_layout != WAVE_X_ROUND)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": row_sq goes with x_layout WAVE_X_ROUND (x = wave_attn_chain's o)");
  if (row_sq && (reinterpret_cast<uintptr_t>(row_sq) & 3u) != 0)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": row_sq must be 4-byte aligned");
  const int64_t D = static_cast<int64_t>(cache->heads) * cache->head_dim;
  if (D % 128 != 0) return set_error(WAVE_ERR_UNSUPPORTED, f + ": heads * head_dim must be a multiple of 128");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": workspace must be non-null and 256-byte aligned");
  if (workspace_bytes < static_cast<size_t>(p.round_q_rows[round]) * sizeof(float))
    return set_error(WAVE_ERR_CAPACITY, f + ": workspace smaller than qkv_project_workspace()");
  const int32_t n0 = p.round_node_begin[round], n1 = p.round_node_begin[round + 1];
  const int32_t row_tiles = (cache->lpad + wave::kProjTileRows - 1) / wave::kProjTileRows;
  const int32_t col_tiles = static_cast<int32_t>(3 * D / wave::kProjTileCols);
  static_assert(wave::kProjTileCols == 128, "D must be a multiple of the column tile");
  if (static_cast<int64_t>(n1 - n0) * row_tiles * col_tiles > INT32_MAX ||
      static_cast<int64_t>(p.params.chunk_len) * D * 2 > UINT32_MAX)
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": too many workgroups or chunk rows too large");
  const int32_t* desc = static_cast<const int32_t*>(d_desc);
  wave::ProjArgs a{};
  a.nodes = desc + p.desc[8];
  a.ctx = desc + p.desc[9];
  a.node_begin = n0;
  a.num_nodes = n1 - n0;
  a.max_rows = p.params.chunk_len;
  a.row_tiles = row_tiles;
  a.col_tiles = col_tiles;
  a.x = x;
  a.x_chunk = x_layout == WAVE_X_CHUNK;
  a.chunk_rows = p.params.chunk_len;
  a.w = w;
  a.model_dim = static_cast<int32_t>(D);
  a.heads = cache->heads;
  a.head_dim = cache->head_dim;
  a.lpad = cache->lpad;
  a.k = cache->k;
  a.vt = cache->vt;
  a.q = q;
  a.row_scale = static_cast<float*>(workspace);
  a.row_sq = row_sq;
  const hipError_t e = wave::launch_qkv_project(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, f + ": " + hipGetErrorString(e));
  return ok();
}

int32_t chain_store(const wave_plan_t* plan, const void* d_desc, int32_t round, int32_t model_dim,
                    const void* o, void* state, void* stream) {
  const std::string f("chain_store");
  if (!plan || !d_desc || !o || !state) return set_error(WAVE_ERR_INVALID_ARG, f + ": null argument");
  const wave::Plan& p = plan->p;
  if (round < 0 || round >= p.num_rounds()) return set_error(WAVE_ERR_INVALID_ARG, f + ": round out of range");
  const int32_t rc = chain_plan_check(p, f);
  if (rc != WAVE_OK) return rc;
  if (model_dim < 8 || model_dim % 8 != 0)
    return set_error(WAVE_ERR_INVALID_ARG, f + ": model_dim must be a positive multiple of 8");
  if (!aligned16(o) || !aligned16(state) || !aligned16(d_desc))
    return set_error(WAVE_ERR_UNSUPPORTED, f + ": o, state and the descriptor must be 16-byte aligned");
  const int64_t n16 = static_cast<int64_t>(p.params.chunk_len) * model_dim / 8;
  if ((n16 + 255) / 256 > INT32_MAX) return set_error(WAVE_ERR_UNSUPPORTED, f + ": chunk too large");
  wave::StoreArgs a{};
  a.nodes = static_cast<const int32_t*>(d_desc) + p.desc[8];
  a.node_begin = p.round_node_begin[round];
  a.num_nodes = p.round_node_begin[round + 1] - a.node_begin;
  a.max_rows = p.params.chunk_len;
  a.model_dim = model_dim;
  a.chunk_rows = p.params.chunk_len;
  a.o = o;
  a.state = state;
  const hipError_t e = wave::launch_chain_store(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(WAVE_ERR_HIP, f + ": " + hipGetErrorString(e));
  return ok();
}

const char* wave_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
