// Decode dispatch: fills the kernel arguments from the validated ABI
// structures, carves the caller's workspace into arrival counters and
// split-K partials, and launches the selected decode kernel.
#include <cmath>

#include "kvq2_decode_common.h"

namespace kvq {

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);
int launch_decode_mfma(const DecodeArgs& a, int batch, void* stream);

int launch_decode(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                  const kvq_cache& cache, int32_t batch, const int32_t* seq_len,
                  int32_t /*max_seq_len*/, const uint16_t* q, float* out, void* workspace,
                  const DecodePlan& plan, DecodeKernel which, void* stream) {
  DecodeArgs a{};
  a.R_K = layer.R_K;
  a.R_V = layer.R_V;
  a.pool = cache.pool;
  a.num_pages = cache.num_pages;
  a.sink = cache.sink;
  a.recent = cache.recent;
  a.block_table = cache.block_table;
  a.bt_stride = cache.bt_stride;
  a.n_q_heads = d.n_q_heads;
  a.n_kv_heads = d.n_kv_heads;
  a.group = d.n_q_heads / d.n_kv_heads;
  a.page_size = d.page_size;
  a.n_sink = d.n_sink;
  a.n_recent = d.n_recent;
  a.alpha = sm_scale * kLog2e;
  // Every V scale is fp16((max - min) / 3) of values clipped to +-clip_V, so
  // s_V <= (2/3) clip_V (1 + 2^-11); sigma_v maps that bound to <= 1.
  a.log2_sigma_v = -static_cast<int>(
      std::ceil(std::log2(static_cast<double>(layer.clip_V) * (2.0 / 3.0) * 1.001)));
  a.sigma_v = std::ldexp(1.0f, a.log2_sigma_v);
  const int cpp = d.page_size / kChunkTokens;
  a.log2_cpp = cpp == 1 ? 0 : cpp == 2 ? 1 : 2;
  a.page_bytes = int64_t(d.n_kv_heads) * cpp * kChunkBytes;
  a.seq_len = seq_len;
  a.q = q;
  a.out = out;
  a.tickets = static_cast<int32_t*>(workspace);
  a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ticket_bytes);
  a.n_split_int2 = plan.n_split_int2;
  a.n_split = plan.n_split;
  if (which == kDecodeValu) return launch_decode_valu(a, batch, stream);
  return launch_decode_mfma(a, batch, stream);
}

}  // namespace kvq
