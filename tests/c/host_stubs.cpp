// Host-only stand-ins for the HIP runtime calls and kernel launchers that the
// C ABI shim uses, so that the planner, the tail-balancing model and the shim
// can be built with g++ under AddressSanitizer / UndefinedBehaviorSanitizer
// and exercised without a GPU.  Each launcher checks the invariants its
// kernel relies on and records the launch.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "kernels.hpp"

namespace stub {
long launches = 0;
int compute_units = 256;
}  // namespace stub

#define STUB_CHECK(cond)                                                   \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "stub check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__); \
      std::abort();                                                        \
    }                                                                      \
  } while (0)

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = stub::compute_units;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace wave {

static char g_scratch[4096];

hipError_t scratch_buffer(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t) {
  STUB_CHECK(a.num_writes >= 0 && a.lpad % 64 == 0 && a.heads >= 1);
  if (a.num_writes > 0) STUB_CHECK(a.writes && a.k && a.vt && a.k_src && a.v_src);
  ++stub::launches;
  return hipSuccess;
}

hipError_t launch_wave_attn(const AttnArgs& a, hipStream_t) {
  STUB_CHECK(a.num_work >= 0 && a.work_begin >= 0 && a.heads >= 1);
  STUB_CHECK(a.num_direct >= 0 && a.num_direct <= a.num_work);
  STUB_CHECK(a.num_splits >= 1 && a.tail_splits >= 1);
  if (a.num_splits > 1 || a.num_direct < a.num_work) STUB_CHECK(a.part_o && a.part_lse && a.part_rows > 0);
  STUB_CHECK(a.q && a.o && a.k && a.vt && a.nodes && a.ctx && a.work);
  ++stub::launches;
  return hipSuccess;
}

hipError_t launch_qkv_project(const ProjArgs& a, hipStream_t) {
  STUB_CHECK(a.num_nodes >= 0 && a.model_dim % 128 == 0 && a.row_scale && a.x && a.w && a.q);
  if (a.row_sq) STUB_CHECK(a.x_chunk == 0);
  ++stub::launches;
  return hipSuccess;
}

hipError_t launch_chain_store(const StoreArgs& a, hipStream_t) {
  STUB_CHECK(a.num_nodes >= 0 && a.model_dim % 8 == 0 && a.o && a.state);
  ++stub::launches;
  return hipSuccess;
}

}  // namespace wave
