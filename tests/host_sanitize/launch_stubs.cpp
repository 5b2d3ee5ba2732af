// Stand-ins for the HIP launchers of libkvq2, so that its host code
// (validation, planning, calibration) builds and runs with the host address
// and undefined-behaviour sanitizers and no GPU.  Each records what it was
// asked to launch; none touches device memory.
#include <cstdio>

#include "kvq2_hqmq_internal.h"
#include "kvq2_internal.h"

namespace kvq {

int g_launches = 0;             // launches requested so far
size_t g_last_ws_bytes = 0;     // plan size of the last decode launch

int launch_quantize_append(const kvq_dims&, float, const kvq_layer&, const kvq_cache&, int32_t,
                           const int32_t*, const int32_t*, int32_t total_new, const uint16_t*,
                           const uint16_t*, void*) {
  ++g_launches;
  return total_new > 0 ? 0 : 1;
}

int launch_decode_step(const kvq_dims&, float, const kvq_layer&, const kvq_cache&, int32_t,
                       const int32_t*, const int32_t*, int32_t total_new, const uint16_t*,
                       const uint16_t*, const int32_t*, int32_t, const uint16_t*, float*, void*,
                       const DecodePlan& plan, void*) {
  ++g_launches;
  g_last_ws_bytes = plan.total_bytes;
  return total_new > 0 && total_new <= kStepAppendMax ? 0 : 1;
}

int launch_decode(const kvq_dims&, float, const kvq_layer&, const kvq_cache&, int32_t,
                  const int32_t*, int32_t, const uint16_t*, float*, void*,
                  const DecodePlan& plan, DecodeKernel, void*, int32_t, int32_t, int32_t,
                  const kvq_prefix_groups*) {
  ++g_launches;
  g_last_ws_bytes = plan.total_bytes;
  return 0;
}

int static_scratch(void** ptr) {
  static unsigned char fake[16] __attribute__((aligned(256)));
  *ptr = fake;
  return 0;
}

int launch_zero_words(void*, size_t bytes, void*) { return bytes % 4 == 0 ? 0 : 1; }

const char* hip_error_name(int err) { return err ? "stub launch error" : "no error"; }

namespace hqmq {

int launch_append(const kvq_hqmq_dims&, const kvq_hqmq_layer&, const kvq_hqmq_cache&, int32_t,
                  const int32_t*, const int32_t*, int32_t total_new, const uint16_t*,
                  const uint16_t*, void*, void*) {
  ++g_launches;
  return total_new > 0 ? 0 : 1;
}

int launch_decode(const kvq_hqmq_dims&, const kvq_hqmq_layer&, const kvq_hqmq_cache&, int32_t,
                  const int32_t*, const uint16_t*, float*, void*, const DecodePlan& plan, void*) {
  ++g_launches;
  g_last_ws_bytes = plan.partial_bytes;
  return plan.n_split >= 1 && plan.n_pass >= 1 ? 0 : 1;
}

}  // namespace hqmq

}  // namespace kvq
