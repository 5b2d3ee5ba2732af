// Internal declarations shared by the libkvq2 sources (host validation,
// calibration and the HIP launchers).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvq2.h"

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kChunkTokens = 16;       // a page is a whole number of 16-token chunks
constexpr int kChunkBytes = 1152;      // 512 K codes + 512 V codes + 64 + 64 params
// With ng (scale, zero) pairs per vector (quantization groups of 128 / ng
// channels) a chunk holds 1024 code bytes and 2 x 16 x ng x 4 param bytes:
// K group k of slot t at 1024 + 4 (t ng + k), V at 1024 + 64 ng + 4 (t ng + k).
constexpr int chunk_bytes_for(int ng) { return 1024 + 128 * ng; }
constexpr int kKCodesOff = 0;
constexpr int kVCodesOff = 512;
constexpr int kKParamsOff = 1024;
constexpr int kVParamsOff = 1088;
constexpr int kMaxGroup = 16;          // query heads per KV head supported
constexpr float kMaxClip = 16384.0f;   // keeps 2c/3 and c inside fp16 range
constexpr int kPartialStride = 132;    // floats per (split, query head) partial:
                                       // m, l, 2 pad, o'[128]
constexpr int kQStride = 132;          // floats per rotated query: q'[128], sum(q'),
                                       // f16 scaling exponent, 2 pad
// u32 words per (b, h) of the QK operand block: [64 lanes][16 dwords] of
// operand, then [64 lanes][4] lane constants (qscale, then the sum of q'
// over the lane's quantization group in each of up to two column sets,
// divided by qscale).
constexpr int kBqOperandWords = 64 * 16;
constexpr int kBqWords = kBqOperandWords + 64 * 4;

// 16-token chunks per tile of the MFMA decode for head-group width gp (2, 4
// or 8): the QK tile's 16 columns hold (chunk, f16 hi/lo, head), so a tile
// spans 16 / (2 gp) chunks; the eight-head tile fills all 16 columns with
// one chunk and takes two chunks per tile (two QK products, one PV product
// over both).
constexpr int chunks_per_tile(int gp) { return gp >= 8 ? 2 : 16 / (2 * gp); }

// Resolved decode geometry shared by the workspace query and the launch.
struct DecodePlan {
  int n_split_int2;   // VALU decode: even splits per (sequence, KV head) of its INT2 chunks
  int n_split;        // VALU decode: n_split_int2 + 1 (the last one takes the bf16 segments)
  size_t ticket_bytes;
  size_t qrot_bytes;    // rotated queries [B][Hq][kQStride] fp32
  size_t bq_bytes;      // QK MFMA operand per (b, h): kBqWords u32
  int piece_cost;       // MFMA decode: virtual tiles charged per (b, h) piece start
  int n_tok_slices;     // MFMA decode: 64-token slices of the token-by-token list
  int64_t tok_slot0;    // MFMA decode: first partial slot of those slices
  size_t prefix_bytes;   // MFMA decode: per-sequence tile prefix [B + 1] int32
  // MFMA decode with shared-prefix groups (0 groups otherwise)
  int n_groups;
  int n_members;
  int n_items_max;      // row-set items: Hkv x sum over groups of ceil(members / 4), bounded
  int rs_cost;          // virtual tiles per row-set tile
  size_t group_bytes;   // per-sequence skip / member / group [3][B], group rows, item ranges
  int64_t rs_slot0;     // first partial slot of the row-set pieces (4 per range and item)
  size_t partial_bytes;
  size_t total_bytes;
};

// Shared-prefix groups of the MFMA decode: grp_info row width and the
// largest number of groups.
constexpr int kGrpInfo = 8;
constexpr int kMaxPrefixGroups = 256;
constexpr int kMaxPrefixMembers = 1024;

// Upper bound of the MFMA decode's work-group count (resident work-groups of
// the device, 256 CUs x 4); its partial slots number kChainGroups + B * Hkv,
// followed by B * Hkv * n_tok_slices slots of the token-list slices.
constexpr int kChainGroups = 1024;
// Fixed cost of one more piece of the MFMA decode (its prologue, the first
// tile's latency, the partial store and the combine), in 16-token chunks of
// streaming: about 15 us of one work-group's stream.  A work-group of the
// eight-head kernel streams about twice as many chunks per us; on the
// 64-sequence G = 8 batch with a shared prefix, 150 chunks measured best in
// sustained decode (395 us against 398 at 200 and 406 at 300).
constexpr int kPieceCostChunks = 80;
constexpr int kPieceCostChunksG8 = 150;
// Virtual tiles charged per tile of a shared-prefix row-set item: its
// work-group's four waves all attend that tile (for four members), so it
// takes about as long as the four tiles a plain work-group streams
// meanwhile (64-sequence G = 8 batch with a 16K shared prefix: 331.8, 327.1,
// 329.8 us per decode at 3, 4, 5).
constexpr int kRowSetCost = 4;

// Plan of a decode with n_query queries per sequence (1 for decode; M for
// multi-query attention): its rows per (sequence, KV head) are
// n_query * Hq / Hkv.
DecodePlan make_decode_plan(const kvq_dims& d, int32_t batch, int32_t max_seq_len,
                            int32_t n_query = 1, const kvq_prefix_groups* groups = nullptr);

// Whether the decode of these dims takes shared-prefix groups (the
// matrix-core kernel with one (scale, zero) pair per vector and at most 8
// query heads per KV head); otherwise a prefix-aware call decodes every
// sequence on its own.
bool prefix_groups_supported(const kvq_dims& d);

// Tuning constants of the MFMA decode, read once per process from the
// environment (KVQ_PIECE_COST, KVQ_ROUND_WEIGHTS, KVQ_XCD_WEIGHTS,
// KVQ_ROWSET_COST, KVQ_ADAPT) with the
// measured defaults.  Range weights are clamped so that the largest is at
// most four times the smallest: with at least four virtual tiles per range
// on average (the cut's precondition) no weighted range is then empty.
struct DecodeTuning {
  int piece_cost[2];        // chunks charged per piece start: [G <= 4, G = 8]
  int round_weight[2][4];   // [G <= 4, G = 8][dispatch round], 1/1024 units
  int xcd_weight[2][2];     // [G <= 4, G = 8][even, odd XCD]
  int rowset_cost;          // virtual tiles charged per tile of a shared-prefix row-set item
  int adapt;                // 1: range weights self-calibrate from measured durations
};
const DecodeTuning& decode_tuning();

// Kernel variants of the decode path.
enum DecodeKernel { kDecodeMfma = 0, kDecodeValu = 1 };
DecodeKernel selected_decode_kernel(const kvq_dims& d);

// Launchers (defined in the .hip sources).  They return a hipError_t value
// (0 = success) so that the host validation code needs no HIP headers.
int launch_quantize_append(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                           const kvq_cache& cache, int32_t batch, const int32_t* start_pos,
                           const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                           const uint16_t* v_new, void* stream);

// Appends of at most this many new tokens in all run the one-token-per-wave
// step kernel (decode steps), and can be fused with the decode pre-pass.
constexpr int kStepAppendMax = 1024;

// Fused decode step (append work-groups in the decode pre-pass launch); the
// MFMA decode and 0 < total_new <= kStepAppendMax only (returns -1 otherwise,
// before any launch).
int launch_decode_step(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                       const kvq_cache& cache, int32_t batch, const int32_t* start_pos,
                       const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                       const uint16_t* v_new, const int32_t* seq_len, int32_t max_seq_len,
                       const uint16_t* q, float* out, void* workspace, const DecodePlan& plan,
                       void* stream);

int launch_decode(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                  const kvq_cache& cache, int32_t batch, const int32_t* seq_len,
                  int32_t max_seq_len, const uint16_t* q, float* out, void* workspace,
                  const DecodePlan& plan, DecodeKernel which, void* stream,
                  int32_t n_query = 1, int32_t query_base = 0, int32_t query_count = 1,
                  const kvq_prefix_groups* groups = nullptr);

// Queries per launch of a multi-query attention of M queries per sequence:
// the matrix-core decode takes at most 8 rows (queries x Hq / Hkv) per pass
// over the pages, the VALU decode 16.
int multi_query_pass(const kvq_dims& d, int32_t n_query, DecodeKernel which);

// The library-owned decode scratch of kvq_decode_attention_noalloc: a
// file-scope device array of kStaticScratchBytes per GPU.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// Device address of the current device's scratch (resolved once per device
// with hipGetSymbolAddress); returns a hipError_t value.
int static_scratch(void** ptr);
// Device address of the current device's self-calibrating range-weight
// states (kFbStates x kFbWords words, zero at load; resolved once per
// device); returns a hipError_t value.
int decode_feedback(void** ptr);
// Zero `bytes` (a multiple of 4) at device address p with a fill kernel
// (no memset node, so the call can be captured in a HIP graph).
int launch_zero_words(void* p, size_t bytes, void* stream);

const char* hip_error_name(int err);
void set_last_error(const char* msg);

}  // namespace kvq
