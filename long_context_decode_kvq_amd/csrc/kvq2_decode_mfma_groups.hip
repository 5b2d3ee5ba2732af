// Matrix-core decode kernels for quantization groups of 64 or 32 channels
// (two or four (s, z) pairs per vector; kvq2_decode_mfma_kernels.h), for up
// to four rows per (sequence, KV head), built as a code object of their own.
#include "kvq2_decode_mfma_kernels.h"

namespace kvq {
namespace {

template <int GP, int NG>
int per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<GP, NG>, 256, 0) !=
          hipSuccess || n <= 0)
    return 1;
  return n;
}

}  // namespace

// Work-groups of decode_mfma_kernel<gp, ng> one CU holds at once.
int decode_mfma_groups_per_cu(int gp, int ng) {
  if (gp == 2) return ng == 2 ? per_cu<2, 2>() : per_cu<2, 4>();
  return ng == 2 ? per_cu<4, 2>() : per_cu<4, 4>();
}

// The streaming kernel of a decode with a.ng = 2 or 4 and a.gp = 2 or 4
// (grid: the streaming work-groups, then the token-list slices).
int launch_decode_mfma_groups(const DecodeArgs& a, unsigned grid, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.gp == 2) {
    if (a.ng == 2) hipLaunchKernelGGL((decode_mfma_kernel<2, 2>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<2, 4>), dim3(grid), dim3(256), 0, st, a);
  } else {
    if (a.ng == 2) hipLaunchKernelGGL((decode_mfma_kernel<4, 2>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((decode_mfma_kernel<4, 4>), dim3(grid), dim3(256), 0, st, a);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
