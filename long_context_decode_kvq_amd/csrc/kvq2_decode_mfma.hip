// Placeholder until the MFMA decode kernel lands: routes to the VALU kernel.
#include "kvq2_decode_common.h"

namespace kvq {
int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);
int launch_decode_mfma(const DecodeArgs& a, int batch, void* stream) {
  return launch_decode_valu(a, batch, stream);
}
}  // namespace kvq
