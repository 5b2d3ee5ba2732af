// libkvq2 host side: argument validation, decode planning and the public
// entry points of the online path.  Validation runs before any HIP call so
// that every error is reported without touching the device.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kvq2_internal.h"

namespace kvq {

namespace {

thread_local std::string g_last_error;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks common to the online calls.
int check_dims(const kvq_dims* d) {
  if (d == nullptr) return KVQ_ERR_ARG;
  if (d->head_dim != kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (d->n_kv_heads < 1 || d->n_q_heads < 1) return KVQ_ERR_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return KVQ_ERR_ARG;
  if (d->n_q_heads / d->n_kv_heads > kMaxGroup) return KVQ_ERR_UNSUPPORTED;
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64) return KVQ_ERR_UNSUPPORTED;
  if (d->n_sink < 0 || d->n_recent < 1) return KVQ_ERR_ARG;
  if (!std::isfinite(d->sm_scale)) return KVQ_ERR_ARG;
  if (d->quant_group != 0 && d->quant_group != 32 && d->quant_group != 64 &&
      d->quant_group != kHeadDim)
    return KVQ_ERR_UNSUPPORTED;
  if (d->hadamard_block != 0 && d->hadamard_block != 32 && d->hadamard_block != 64 &&
      d->hadamard_block != kHeadDim)
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int check_layer(const kvq_layer* l) {
  if (l == nullptr || l->R_K == nullptr || l->R_V == nullptr) return KVQ_ERR_ARG;
  if (!aligned16(l->R_K) || !aligned16(l->R_V)) return KVQ_ERR_ARG;
  for (float c : {l->clip_K, l->clip_V})
    if (!(c > 0.0f) || !(c <= kMaxClip)) return KVQ_ERR_ARG;   // also rejects NaN
  return KVQ_OK;
}

int check_cache(const kvq_dims* d, const kvq_cache* c) {
  if (c == nullptr || c->pool == nullptr || c->recent == nullptr || c->block_table == nullptr)
    return KVQ_ERR_ARG;
  if (d->n_sink > 0 && c->sink == nullptr) return KVQ_ERR_ARG;
  if (!aligned16(c->pool) || !aligned16(c->recent) || !aligned16(c->block_table)) return KVQ_ERR_ARG;
  if (c->sink != nullptr && !aligned16(c->sink)) return KVQ_ERR_ARG;
  if (c->num_pages < 1 || c->bt_stride < 1) return KVQ_ERR_ARG;
  return KVQ_OK;
}

float resolved_scale(const kvq_dims* d) {
  return d->sm_scale > 0.0f ? d->sm_scale : 1.0f / std::sqrt(static_cast<float>(kHeadDim));
}

int env_int(const char* name, int fallback) {
  const char* s = std::getenv(name);
  if (s == nullptr || *s == '\0') return fallback;
  return std::atoi(s);
}

}  // namespace

void set_last_error(const char* msg) { g_last_error = msg ? msg : ""; }

namespace {

// Range weights of the MFMA decode's cut.  The resident work-groups of one
// CU do not stream at one rate: the instruction arbiter favours the oldest
// waves, so on the 28 x 100000-token batch (four work-groups per CU) equal
// ranges stream at 2.88, 2.68, 2.45 and 2.31 tiles/us from the first to the
// fourth dispatched, and on the 64-sequence G = 8 batch (three per CU) the
// third round ends ~29 us after the first.  The round weights, a little
// steeper than those rates, gave the shortest sustained decode in A/B runs
// (28 x 100000: 334 -> 328 us per step; 64-sequence G = 8: 403 -> 392 us).
// A per-XCD weight is supported but left even: one MI355X showed odd XCDs
// ending 10-15 us late, another ran fastest with even weights (decode call
// 298 us even against 304-311 us with a 1060/988 or 1100/950 skew), so the
// skew belongs to the machine, not to the kernel.
DecodeTuning read_tuning() {
  DecodeTuning t = {{kPieceCostChunks, kPieceCostChunksG8},
                    {{1230, 1100, 940, 830}, {1120, 1024, 930, 1024}},
                    {{1024, 1024}, {1024, 1024}},
                    kRowSetCost,
                    1};
  t.rowset_cost = std::min(std::max(env_int("KVQ_ROWSET_COST", kRowSetCost), 1), 16);
  t.adapt = env_int("KVQ_ADAPT", 1) != 0 ? 1 : 0;
  const int pc = env_int("KVQ_PIECE_COST", -1);
  if (pc >= 0) t.piece_cost[0] = t.piece_cost[1] = std::min(pc, 4096);
  for (int k = 0; k < 2; ++k) {
    if (const char* s = std::getenv("KVQ_ROUND_WEIGHTS"))
      std::sscanf(s, "%d,%d,%d,%d", &t.round_weight[k][0], &t.round_weight[k][1],
                  &t.round_weight[k][2], &t.round_weight[k][3]);
    if (const char* s = std::getenv("KVQ_XCD_WEIGHTS"))
      std::sscanf(s, "%d,%d", &t.xcd_weight[k][0], &t.xcd_weight[k][1]);
    // round x XCD products within a factor of four of each other
    int rmax = 1, xmax = 1;
    for (int r = 0; r < 4; ++r) rmax = std::max(rmax, std::min(t.round_weight[k][r], 4096));
    for (int x = 0; x < 2; ++x) xmax = std::max(xmax, std::min(t.xcd_weight[k][x], 4096));
    for (int r = 0; r < 4; ++r)
      t.round_weight[k][r] = std::min(std::max(t.round_weight[k][r], (rmax + 1) / 2), rmax);
    for (int x = 0; x < 2; ++x)
      t.xcd_weight[k][x] = std::min(std::max(t.xcd_weight[k][x], (xmax + 1) / 2), xmax);
  }
  return t;
}

}  // namespace

const DecodeTuning& decode_tuning() {
  static const DecodeTuning t = read_tuning();   // thread-safe one-time initialisation
  return t;
}

DecodeKernel selected_decode_kernel(const kvq_dims& d) {
  // KVQ_DECODE_KERNEL=valu selects the plain VALU kernel (kept as the
  // measured comparison point for the MFMA kernel); default is MFMA.  The
  // MFMA kernel takes quantization groups narrower than 128 channels for up
  // to four query heads per KV head; wider groups of heads then take the
  // VALU kernel.
  const char* s = std::getenv("KVQ_DECODE_KERNEL");
  if (s != nullptr && std::strcmp(s, "valu") == 0) return kDecodeValu;
  if (d.quant_group != 0 && d.quant_group != kHeadDim && d.n_q_heads / d.n_kv_heads > 4)
    return kDecodeValu;
  return kDecodeMfma;
}

bool prefix_groups_supported(const kvq_dims& d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const bool narrow = d.quant_group != 0 && d.quant_group != kHeadDim;
  return selected_decode_kernel(d) == kDecodeMfma && G <= 8 && !narrow;
}

int multi_query_pass(const kvq_dims& d, int32_t n_query, DecodeKernel which) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const bool narrow = d.quant_group != 0 && d.quant_group != kHeadDim;
  const int rows = (which == kDecodeMfma && G <= 8) ? (narrow ? 4 : 8) : kMaxGroup;
  return std::max(1, std::min<int>(n_query, rows / G));
}

DecodePlan make_decode_plan(const kvq_dims& d, int32_t batch, int32_t max_seq_len,
                            int32_t n_query, const kvq_prefix_groups* groups) {
  DecodePlan p{};
  const int64_t int2_end = std::max<int64_t>(d.n_sink, int64_t(max_seq_len) - d.n_recent);
  const int64_t first_chunk = d.n_sink / kChunkTokens;
  const int64_t last_chunk = (int2_end + kChunkTokens - 1) / kChunkTokens;   // exclusive
  const int64_t n_chunks = int2_end > d.n_sink ? last_chunk - first_chunk : 0;
  const int64_t heads = int64_t(batch) * d.n_kv_heads;
  // VALU decode: even splits, about two work-groups per resident slot of the
  // GPU (2048 = 256 CUs x 4 x 2), but no split shorter than 256 chunks (4096
  // tokens): the split prologue and its share of the combine are paid per
  // split.
  int64_t nb = (2048 + heads - 1) / std::max<int64_t>(heads, 1);
  nb = std::min<int64_t>(nb, std::max<int64_t>(1, n_chunks / 256));
  nb = std::max<int64_t>(1, std::min<int64_t>(nb, 512));
  if (n_chunks == 0) nb = 1;
  p.n_split_int2 = static_cast<int>(nb);
  // The MFMA decode deals the token-by-token list out over its INT2 items;
  // the VALU decode (also used for G > 8) gives it a work-group of its own.
  const int G = (d.n_q_heads / d.n_kv_heads) * n_query;   // rows per (b, h)
  const bool own_token_item = selected_decode_kernel(d) == kDecodeValu || G > 8;
  p.n_split = p.n_split_int2 + (own_token_item ? 1 : 0);
  // arrival tickets [B * Hkv] of the VALU decode's last-arrival combine
  p.ticket_bytes = ((size_t(heads) * sizeof(int32_t) + 255) / 256) * 256;
  p.qrot_bytes = size_t(heads) * G * kQStride * sizeof(float);
  p.bq_bytes = size_t(heads) * kBqWords * sizeof(uint32_t);
  // tile prefix [B + 1], range starts [kChainGroups + 1], pair ranges [B Hkv]
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  p.prefix_bytes = r256((size_t(batch) + 1) * sizeof(int32_t)) +
                   r256((size_t(kChainGroups) + 1) * sizeof(int32_t)) +
                   r256(size_t(heads) * sizeof(int32_t));
  // The MFMA decode cuts all (b, h) tiles into at most kChainGroups equal
  // ranges: a work-group leaves one partial per (b, h) it touches, in slot
  // group + b * Hkv + h (unique: the (group, pair) overlaps form a monotone
  // path), so kChainGroups + B * Hkv slots suffice.
  if (!own_token_item) {
    // The token-by-token list of a sequence: the sink, at most 15 INT2
    // positions before the first whole chunk, at most 16 npt - 1 after the
    // last whole tile, and the recent window.
    const int gp = G <= 2 ? 2 : G <= 4 ? 4 : 8;
    const int npt = chunks_per_tile(gp);
    const int64_t max_list = int64_t(d.n_sink) + 15 + (16 * npt - 1) + d.n_recent;
    p.n_tok_slices = static_cast<int>((max_list + 63) / 64);
    p.tok_slot0 = int64_t(kChainGroups) + heads;
    p.piece_cost = decode_tuning().piece_cost[gp == 8 ? 1 : 0] / npt;
  }
  size_t slots = own_token_item
                     ? size_t(heads) * p.n_split
                     : size_t(kChainGroups) + size_t(heads) * (1 + p.n_tok_slices);
  // Shared-prefix groups: row-set items (Hkv per row set of four members;
  // sum of ceil(n_j / 4) <= (n_members + 3 n_groups) / 4), four partial slots
  // per (range, item) overlap, and the per-sequence and per-group tables.
  if (groups != nullptr && groups->n_groups > 0 && !own_token_item && n_query == 1 &&
      prefix_groups_supported(d)) {
    p.n_groups = groups->n_groups;
    p.n_members = groups->n_members;
    p.n_items_max = static_cast<int>(int64_t(d.n_kv_heads) *
                                     ((int64_t(groups->n_members) + 3 * groups->n_groups) / 4));
    p.rs_cost = decode_tuning().rowset_cost;
    p.group_bytes = 3 * r256(size_t(batch) * sizeof(int32_t)) +
                    r256(size_t(groups->n_groups) * kGrpInfo * sizeof(int32_t)) +
                    r256(size_t(p.n_items_max) * sizeof(int32_t));
    p.rs_slot0 = int64_t(slots);
    slots += 4 * (size_t(kChainGroups) + size_t(p.n_items_max));
  }
  p.partial_bytes = slots * G * kPartialStride * sizeof(float);
  p.total_bytes = p.ticket_bytes + p.qrot_bytes + p.bq_bytes + p.prefix_bytes + p.group_bytes +
                  p.partial_bytes;
  return p;
}

}  // namespace kvq

using namespace kvq;

namespace {

// Argument checks of an append (before any HIP call); KVQ_OK with
// *nothing = true when there is nothing to append.
int check_append(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                 int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                 int32_t total_new, int32_t max_new, const uint16_t* k_new,
                 const uint16_t* v_new, bool* nothing) {
  int rc = check_dims(dims);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_layer(layer)) != KVQ_OK) return rc;
  if ((rc = check_cache(dims, cache)) != KVQ_OK) return rc;
  if (batch < 1 || total_new < 0 || max_new < 0 || max_new > total_new) return KVQ_ERR_ARG;
  if (start_pos == nullptr || cu_new == nullptr) return KVQ_ERR_ARG;
  *nothing = total_new == 0;
  if (*nothing) return KVQ_OK;
  if (k_new == nullptr || v_new == nullptr || !aligned16(k_new) || !aligned16(v_new))
    return KVQ_ERR_ARG;
  return KVQ_OK;
}

// Argument checks of a decode other than its workspace (before any HIP
// call); fills the plan.
int check_decode_args(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                      int32_t batch, const int32_t* seq_len, int32_t max_seq_len,
                      const uint16_t* q, float* out, DecodePlan* plan, int32_t n_query = 1) {
  int rc = check_dims(dims);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_layer(layer)) != KVQ_OK) return rc;
  if ((rc = check_cache(dims, cache)) != KVQ_OK) return rc;
  if (batch < 1 || max_seq_len < 0 || seq_len == nullptr) return KVQ_ERR_ARG;
  // multi-query: every query must see the whole INT2 history (M <= W)
  if (n_query < 1 || n_query > dims->n_recent) return KVQ_ERR_ARG;
  if (q == nullptr || out == nullptr || !aligned16(q) || !aligned16(out)) return KVQ_ERR_ARG;
  if (int64_t(max_seq_len) > int64_t(cache->bt_stride) * dims->page_size) return KVQ_ERR_ARG;
  // The MFMA decode counts virtual tiles of the whole batch in 32 bits.
  if (int64_t(batch) * dims->n_kv_heads * (int64_t(max_seq_len) / kChunkTokens + kPieceCostChunksG8 + 2) >=
      (int64_t(1) << 31))
    return KVQ_ERR_UNSUPPORTED;
  *plan = make_decode_plan(*dims, batch, max_seq_len,
                           multi_query_pass(*dims, n_query, selected_decode_kernel(*dims)));
  return KVQ_OK;
}

// Argument checks of a decode with a caller workspace.
int check_decode(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                 int32_t batch, const int32_t* seq_len, int32_t max_seq_len, const uint16_t* q,
                 float* out, void* workspace, size_t workspace_bytes, DecodePlan* plan,
                 int32_t n_query = 1) {
  const int rc =
      check_decode_args(dims, layer, cache, batch, seq_len, max_seq_len, q, out, plan, n_query);
  if (rc != KVQ_OK) return rc;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < plan->total_bytes)
    return KVQ_ERR_WORKSPACE;
  return KVQ_OK;
}

int hip_status(int err) {
  if (err == 0) return KVQ_OK;
  set_last_error(hip_error_name(err));
  return KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_ARG: return "KVQ_ERR_ARG: invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: unsupported shape";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: workspace too small";
    case KVQ_ERR_NUMERIC: return "KVQ_ERR_NUMERIC: numerical failure";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: HIP runtime error";
    default: return "KVQ_ERR_UNKNOWN";
  }
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

int kvq_quantize_append(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                        int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                        int32_t total_new, int32_t max_new, const uint16_t* k_new,
                        const uint16_t* v_new, void* stream) {
  bool nothing = false;
  const int rc = check_append(dims, layer, cache, batch, start_pos, cu_new, total_new, max_new,
                              k_new, v_new, &nothing);
  if (rc != KVQ_OK || nothing) return rc;
  return hip_status(launch_quantize_append(*dims, resolved_scale(dims), *layer, *cache, batch,
                                           start_pos, cu_new, total_new, k_new, v_new, stream));
}

size_t kvq_decode_workspace_bytes(const kvq_dims* dims, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims) != KVQ_OK || batch < 1 || max_seq_len < 0) return 0;
  return make_decode_plan(*dims, batch, max_seq_len).total_bytes;
}

int kvq_decode_attention(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                         int32_t batch, const int32_t* seq_len, int32_t max_seq_len,
                         const uint16_t* q, float* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  DecodePlan plan;
  const int rc = check_decode(dims, layer, cache, batch, seq_len, max_seq_len, q, out, workspace,
                              workspace_bytes, &plan);
  if (rc != KVQ_OK) return rc;
  return hip_status(launch_decode(*dims, resolved_scale(dims), *layer, *cache, batch, seq_len,
                                  max_seq_len, q, out, workspace, plan, selected_decode_kernel(*dims),
                                  stream));
}

// Shared-prefix groups: the host values and that the arrays are given.
static int check_groups(const kvq_prefix_groups* groups) {
  if (groups == nullptr || groups->n_groups < 0 || groups->n_groups > kMaxPrefixGroups ||
      groups->n_members < 0 || groups->n_members > kMaxPrefixMembers)
    return KVQ_ERR_ARG;
  if (groups->n_groups > 0 && (groups->member_start == nullptr || groups->members == nullptr ||
                               groups->prefix_len == nullptr))
    return KVQ_ERR_ARG;
  return KVQ_OK;
}

size_t kvq_decode_prefix_workspace_bytes(const kvq_dims* dims, int32_t batch,
                                         int32_t max_seq_len, const kvq_prefix_groups* groups) {
  if (check_dims(dims) != KVQ_OK || batch < 1 || max_seq_len < 0 || check_groups(groups) != KVQ_OK)
    return 0;
  return make_decode_plan(*dims, batch, max_seq_len, 1, groups).total_bytes;
}

int kvq_decode_prefix_attention(const kvq_dims* dims, const kvq_layer* layer,
                                const kvq_cache* cache, int32_t batch, const int32_t* seq_len,
                                int32_t max_seq_len, const uint16_t* q, float* out,
                                const kvq_prefix_groups* groups, void* workspace,
                                size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  int rc = check_decode_args(dims, layer, cache, batch, seq_len, max_seq_len, q, out, &plan, 1);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_groups(groups)) != KVQ_OK) return rc;
  plan = make_decode_plan(*dims, batch, max_seq_len, 1, groups);
  // the row-set items' virtual tiles are counted in 32 bits too
  if (plan.n_groups > 0 &&
      int64_t(batch) * dims->n_kv_heads * (int64_t(max_seq_len) / kChunkTokens + kPieceCostChunksG8 + 2) +
              int64_t(plan.n_items_max) *
                  (int64_t(plan.rs_cost) * (int64_t(max_seq_len) / kChunkTokens) + kPieceCostChunksG8 + 2) >=
          (int64_t(1) << 31))
    return KVQ_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < plan.total_bytes)
    return KVQ_ERR_WORKSPACE;
  return hip_status(launch_decode(*dims, resolved_scale(dims), *layer, *cache, batch, seq_len,
                                  max_seq_len, q, out, workspace, plan, selected_decode_kernel(*dims),
                                  stream, 1, 0, 1, plan.n_groups > 0 ? groups : nullptr));
}

size_t kvq_decode_multi_workspace_bytes(const kvq_dims* dims, int32_t batch,
                                        int32_t max_seq_len, int32_t n_query) {
  if (check_dims(dims) != KVQ_OK || batch < 1 || max_seq_len < 0 || n_query < 1) return 0;
  const int pass = multi_query_pass(*dims, n_query, selected_decode_kernel(*dims));
  return make_decode_plan(*dims, batch, max_seq_len, pass).total_bytes;
}

int kvq_decode_multi_attention(const kvq_dims* dims, const kvq_layer* layer,
                               const kvq_cache* cache, int32_t batch, const int32_t* seq_len,
                               int32_t max_seq_len, int32_t n_query, const uint16_t* q,
                               float* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  DecodePlan plan;
  const int rc = check_decode(dims, layer, cache, batch, seq_len, max_seq_len, q, out, workspace,
                              workspace_bytes, &plan, n_query);
  if (rc != KVQ_OK) return rc;
  // Passes of at most `pass` queries, each over all pages, in stream order
  // on the one workspace.
  const DecodeKernel which = selected_decode_kernel(*dims);
  const int pass = multi_query_pass(*dims, n_query, which);
  for (int m0 = 0; m0 < n_query; m0 += pass) {
    const int nq = std::min(pass, n_query - m0);
    const DecodePlan p = nq == pass ? plan : make_decode_plan(*dims, batch, max_seq_len, nq);
    const int err = launch_decode(*dims, resolved_scale(dims), *layer, *cache, batch, seq_len,
                                  max_seq_len, q, out, workspace, p, which, stream, nq, m0,
                                  n_query);
    if (err != 0) return hip_status(err);
  }
  return KVQ_OK;
}

int kvq_decode_attention_noalloc(const kvq_dims* dims, const kvq_layer* layer,
                                 const kvq_cache* cache, int32_t batch, const int32_t* seq_len,
                                 int32_t max_seq_len, const uint16_t* q, float* out,
                                 void* stream) {
  // Every argument check of kvq_decode_attention; the workspace this call
  // needs must fit the library's scratch.
  DecodePlan plan;
  int rc = check_decode_args(dims, layer, cache, batch, seq_len, max_seq_len, q, out, &plan);
  if (rc != KVQ_OK) return rc;
  if (plan.total_bytes > kStaticScratchBytes) {
    set_last_error("decode workspace larger than the library scratch of "
                   "kvq_decode_attention_noalloc (64 MiB); use kvq_decode_attention");
    return KVQ_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if ((rc = hip_status(static_scratch(&ws))) != KVQ_OK) return rc;
  // The arrival counters of the VALU decode must start at zero; the scratch
  // keeps whatever the previous call on this GPU left.
  const DecodeKernel which = selected_decode_kernel(*dims);
  if (which == kDecodeValu || dims->n_q_heads / dims->n_kv_heads > 8)
    if ((rc = hip_status(launch_zero_words(ws, plan.ticket_bytes, stream))) != KVQ_OK) return rc;
  return hip_status(launch_decode(*dims, resolved_scale(dims), *layer, *cache, batch, seq_len,
                                  max_seq_len, q, out, ws, plan, which, stream));
}

int kvq_decode_step(const kvq_dims* dims, const kvq_layer* layer, const kvq_cache* cache,
                    int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                    int32_t total_new, int32_t max_new, const uint16_t* k_new,
                    const uint16_t* v_new, const int32_t* seq_len, int32_t max_seq_len,
                    const uint16_t* q, float* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  bool nothing = false;
  int rc = check_append(dims, layer, cache, batch, start_pos, cu_new, total_new, max_new, k_new,
                        v_new, &nothing);
  if (rc != KVQ_OK) return rc;
  DecodePlan plan;
  rc = check_decode(dims, layer, cache, batch, seq_len, max_seq_len, q, out, workspace,
                    workspace_bytes, &plan);
  if (rc != KVQ_OK) return rc;
  const float scale = resolved_scale(dims);
  const int G = dims->n_q_heads / dims->n_kv_heads;
  if (!nothing && total_new <= kStepAppendMax && G <= 8 &&
      selected_decode_kernel(*dims) == kDecodeMfma) {
    return hip_status(launch_decode_step(*dims, scale, *layer, *cache, batch, start_pos, cu_new,
                                         total_new, k_new, v_new, seq_len, max_seq_len, q, out,
                                         workspace, plan, stream));
  }
  // Other shapes: the append, then the decode, in stream order.
  if (!nothing) {
    rc = hip_status(launch_quantize_append(*dims, scale, *layer, *cache, batch, start_pos, cu_new,
                                           total_new, k_new, v_new, stream));
    if (rc != KVQ_OK) return rc;
  }
  return hip_status(launch_decode(*dims, scale, *layer, *cache, batch, seq_len, max_seq_len, q,
                                  out, workspace, plan, selected_decode_kernel(*dims), stream));
}

}  // extern "C"
