// Matrix-core decode kernels for eight query heads per KV head (one
// (scale, zero) pair per vector; kvq2_decode_mfma_kernels.h) and their
// split-K combines, plain and with shared-prefix groups, built as a code
// object of their own.
#include "kvq2_decode_mfma_kernels.h"

namespace kvq {

// Work-groups of decode_mfma_kernel<8, 1> one CU holds at once.
int decode_mfma_g8_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<8, 1>, 256, 0) !=
          hipSuccess || n <= 0)
    return 1;
  return n;
}

// The streaming kernel (grid: the streaming work-groups, then the
// token-list slices) and the combine (per (b, h), or per query head when
// per_head) of an eight-head decode.
void launch_decode_mfma_g8(const DecodeArgs& a, unsigned grid, bool per_head, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL((decode_mfma_kernel<8, 1>), dim3(grid), dim3(256), 0, st, a);
  const dim3 cgrid(a.n_kv_heads, a.batch, per_head ? a.group : 1);
  const dim3 cblock(per_head ? 128 * kHeadCombineParts : combine_threads<8>());
  if (per_head) hipLaunchKernelGGL(combine_head_kernel<8>, cgrid, cblock, 0, st, a);
  else hipLaunchKernelGGL(combine_kernel<8>, cgrid, cblock, 0, st, a);
}

// The same with shared-prefix groups (a.n_groups > 0).
void launch_decode_mfma_g8_prefix(const DecodeArgs& a, unsigned grid, bool per_head,
                                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL((decode_mfma_kernel<8, 1, true>), dim3(grid), dim3(256), 0, st, a);
  const dim3 cgrid(a.n_kv_heads, a.batch, per_head ? a.group : 1);
  const dim3 cblock(per_head ? 128 * kHeadCombineParts : combine_threads<8>());
  if (per_head) hipLaunchKernelGGL((combine_head_kernel<8, true>), cgrid, cblock, 0, st, a);
  else hipLaunchKernelGGL((combine_kernel<8, true>), cgrid, cblock, 0, st, a);
}

}  // namespace kvq
