// libkvq2 host side of the HQMQ codec (include/kvq2_hqmq.h): the codebook
// product, argument validation (before any HIP call), the decode plan and
// the public entry points.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "kvq2_hqmq_internal.h"
#include "kvq2_internal.h"

namespace kvq {
namespace hqmq {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const kvq_hqmq_dims* d) {
  if (d == nullptr) return KVQ_ERR_ARG;
  if (d->head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (d->n_kv_heads < 1 || d->n_q_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return KVQ_ERR_ARG;
  if (d->n_q_heads / d->n_kv_heads > kMaxGroup) return KVQ_ERR_UNSUPPORTED;
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64) return KVQ_ERR_UNSUPPORTED;
  if (d->n_secondary < 1 || d->n_secondary > kMaxSecondary) return KVQ_ERR_UNSUPPORTED;
  if (!std::isfinite(d->sm_scale)) return KVQ_ERR_ARG;
  return KVQ_OK;
}

int check_layer_cache(const kvq_hqmq_layer* l, const kvq_hqmq_cache* c) {
  if (l == nullptr || c == nullptr) return KVQ_ERR_ARG;
  if (l->codebook_K == nullptr || l->codebook_V == nullptr || !aligned16(l->codebook_K) ||
      !aligned16(l->codebook_V))
    return KVQ_ERR_ARG;
  if (c->pool == nullptr || c->block_table == nullptr || !aligned16(c->pool) ||
      !aligned16(c->block_table) || c->num_pages < 1 || c->bt_stride < 1)
    return KVQ_ERR_ARG;
  return KVQ_OK;
}

int hip_status(int err) {
  if (err == 0) return KVQ_OK;
  set_last_error(hip_error_name(err));
  return KVQ_ERR_HIP;
}

// Quaternion (a, b, c, d) product p q, fp64, components summed left to
// right in Hamilton's rule.
void hamilton(const double p[4], const double q[4], double out[4]) {
  const double a1 = p[0], b1 = p[1], c1 = p[2], d1 = p[3];
  const double a2 = q[0], b2 = q[1], c2 = q[2], d2 = q[3];
  out[0] = a1 * a2 - b1 * b2 - c1 * c2 - d1 * d2;
  out[1] = a1 * b2 + b1 * a2 + c1 * d2 - d1 * c2;
  out[2] = a1 * c2 - b1 * d2 + c1 * a2 + d1 * b2;
  out[3] = a1 * d2 + b1 * c2 - c1 * b2 + d1 * a2;
}

// Word p of the binary tetrahedral group: p < 8 the unit along axis p / 2
// with sign (-1)^(p % 2); 8 + m the half-units with component t negative
// iff bit t of m is set.
void primary(int p, double out[4]) {
  for (int t = 0; t < 4; ++t) out[t] = 0.0;
  if (p < 8) {
    out[p / 2] = (p % 2) ? -1.0 : 1.0;
  } else {
    for (int t = 0; t < 4; ++t) out[t] = ((p - 8) >> t & 1) ? -0.5 : 0.5;
  }
}

}  // namespace

float resolved_scale(const kvq_hqmq_dims& d) {
  return d.sm_scale > 0.0f ? d.sm_scale : 1.0f / std::sqrt(static_cast<float>(kHeadDim));
}

int heads_per_pass(int group) { return group <= 4 ? 4 : 8; }

DecodePlan make_plan(const kvq_hqmq_dims& d, int32_t batch, int32_t max_seq_len) {
  DecodePlan p{};
  const int G = d.n_q_heads / d.n_kv_heads;
  p.n_pass = (G + heads_per_pass(G) - 1) / heads_per_pass(G);
  // about eight work-groups per CU over all (sequence, KV head) pairs, but
  // no split shorter than 256 positions
  const int64_t pairs = int64_t(batch) * d.n_kv_heads * p.n_pass;
  int64_t ns = (2048 + pairs - 1) / std::max<int64_t>(pairs, 1);
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, max_seq_len / 256));
  p.n_split = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ns, 1024)));
  p.partial_bytes = size_t(batch) * d.n_kv_heads * p.n_split * G * kPartStride * sizeof(float);
  return p;
}

}  // namespace hqmq
}  // namespace kvq

using namespace kvq;
using namespace kvq::hqmq;

extern "C" {

int kvq_hqmq_codebook(int32_t n_secondary, const float* secondary, float* codebook) {
  if (secondary == nullptr || codebook == nullptr || n_secondary < 1 ||
      n_secondary > kMaxSecondary)
    return KVQ_ERR_ARG;
  for (int i = 0; i < 4 * n_secondary; ++i)
    if (!std::isfinite(secondary[i])) return KVQ_ERR_NUMERIC;
  for (int s = 0; s < n_secondary; ++s) {
    const double q[4] = {secondary[4 * s], secondary[4 * s + 1], secondary[4 * s + 2],
                         secondary[4 * s + 3]};
    for (int p = 0; p < kPrimary; ++p) {
      double pp[4], w[4];
      primary(p, pp);
      hamilton(pp, q, w);
      for (int t = 0; t < 4; ++t) codebook[4 * (kPrimary * s + p) + t] = static_cast<float>(w[t]);
    }
  }
  return KVQ_OK;
}

size_t kvq_hqmq_append_workspace_bytes(const kvq_hqmq_dims* dims, int32_t total_new) {
  if (check_dims(dims) != KVQ_OK || total_new < 0) return 0;
  return kAppendWorkspaceBytes;
}

int kvq_hqmq_append(const kvq_hqmq_dims* dims, const kvq_hqmq_layer* layer,
                    const kvq_hqmq_cache* cache, int32_t batch, const int32_t* start_pos,
                    const int32_t* cu_new, int32_t total_new, int32_t max_new,
                    const uint16_t* k_new, const uint16_t* v_new, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_layer_cache(layer, cache)) != KVQ_OK) return rc;
  if (batch < 1 || total_new < 0 || max_new < 0 || max_new > total_new) return KVQ_ERR_ARG;
  if (start_pos == nullptr || cu_new == nullptr || !aligned16(start_pos) || !aligned16(cu_new))
    return KVQ_ERR_ARG;
  // chunk counts of one role are 32-bit in the median selection
  if (int64_t(total_new) * dims->n_kv_heads * kChunks >= (int64_t(1) << 32)) return KVQ_ERR_ARG;
  if (total_new == 0) return KVQ_OK;
  if (k_new == nullptr || v_new == nullptr || !aligned16(k_new) || !aligned16(v_new))
    return KVQ_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < kAppendWorkspaceBytes)
    return KVQ_ERR_WORKSPACE;
  return hip_status(launch_append(*dims, *layer, *cache, batch, start_pos, cu_new, total_new,
                                  k_new, v_new, workspace, stream));
}

size_t kvq_hqmq_decode_workspace_bytes(const kvq_hqmq_dims* dims, int32_t batch,
                                       int32_t max_seq_len) {
  if (check_dims(dims) != KVQ_OK || batch < 1 || max_seq_len < 0) return 0;
  return make_plan(*dims, batch, max_seq_len).partial_bytes;
}

int kvq_hqmq_decode_attention(const kvq_hqmq_dims* dims, const kvq_hqmq_layer* layer,
                              const kvq_hqmq_cache* cache, int32_t batch, const int32_t* seq_len,
                              int32_t max_seq_len, const uint16_t* q, float* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_layer_cache(layer, cache)) != KVQ_OK) return rc;
  if (batch < 1 || batch > 65535 || max_seq_len < 0) return KVQ_ERR_ARG;
  if (seq_len == nullptr || q == nullptr || out == nullptr || !aligned16(seq_len) ||
      !aligned16(q) || !aligned16(out))
    return KVQ_ERR_ARG;
  const hqmq::DecodePlan plan = make_plan(*dims, batch, max_seq_len);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < plan.partial_bytes)
    return KVQ_ERR_WORKSPACE;
  return hip_status(hqmq::launch_decode(*dims, *layer, *cache, batch, seq_len, q, out, workspace, plan,
                                  stream));
}

}  // extern "C"
