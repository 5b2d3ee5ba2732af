// Matrix-core decode kernels of decodes with shared-prefix groups (their
// row-set items after the (b, h) pieces, and combines that take the
// row-set partials in; kvq2_decode_mfma_kernels.h) for up to four query
// heads per KV head, built as a code object of their own so that plain
// decodes run kernels without that code (eight heads:
// kvq2_decode_mfma_g8.hip).
#include "kvq2_decode_mfma_kernels.h"

namespace kvq {

void launch_decode_mfma_g8_prefix(const DecodeArgs& a, unsigned grid, bool per_head,
                                  void* stream);

// The streaming kernel and the combine (per (b, h), or per query head when
// per_head) of a decode with a.n_groups > 0 and a.ng = 1; gp = 2, 4 or 8.
void launch_decode_mfma_prefix(const DecodeArgs& a, unsigned grid, bool per_head, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 cgrid(a.n_kv_heads, a.batch, per_head ? a.group : 1);
  const dim3 cblock(per_head ? 128 * kHeadCombineParts
                             : (a.gp == 2 ? combine_threads<2>() : combine_threads<4>()));
  if (a.gp == 2) {
    hipLaunchKernelGGL((decode_mfma_kernel<2, 1, true>), dim3(grid), dim3(256), 0, st, a);
    if (per_head) hipLaunchKernelGGL((combine_head_kernel<2, true>), cgrid, cblock, 0, st, a);
    else hipLaunchKernelGGL((combine_kernel<2, true>), cgrid, cblock, 0, st, a);
  } else if (a.gp == 4) {
    hipLaunchKernelGGL((decode_mfma_kernel<4, 1, true>), dim3(grid), dim3(256), 0, st, a);
    if (per_head) hipLaunchKernelGGL((combine_head_kernel<4, true>), cgrid, cblock, 0, st, a);
    else hipLaunchKernelGGL((combine_kernel<4, true>), cgrid, cblock, 0, st, a);
  } else {
    launch_decode_mfma_g8_prefix(a, grid, per_head, stream);
  }
}

}  // namespace kvq
