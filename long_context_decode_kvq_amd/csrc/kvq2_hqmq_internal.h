// libkvq2 internals of the HQMQ codec (include/kvq2_hqmq.h): record layout,
// workspace layouts and the launchers the host entry points call.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvq2.h"
#include "kvq2_hqmq.h"

namespace kvq {
namespace hqmq {

constexpr int kHeadDim = 128;
constexpr int kChunks = 32;             // quaternion chunks of 4 channels per vector
constexpr int kPrimary = 24;            // binary tetrahedral group 2T
constexpr int kMaxSecondary = 10;       // 24 S <= 240 words: one index byte
constexpr int kMaxWords = kPrimary * kMaxSecondary;
constexpr int kMaxKept = 3;             // fp16 chunks per record
constexpr int kRadiusLevels = 255;
constexpr int kRecordBytes = 96;
constexpr int kTokenBytes = 2 * kRecordBytes;
constexpr int kIdxOff = 0, kRadOff = 32, kRmaxOff = 64, kFlagsOff = 68, kKeptOff = 72;
constexpr int kMaxGroup = 16;

// Append workspace: the lower median of each role's chunk norms is selected
// by three histogram passes over the bits of the (non-negative) fp32 norms:
// bits 31..21 (2048 bins), 20..10 (2048), 9..0 (1024).
constexpr int kHistBins = 2048;
struct SelectState {
  uint32_t prefix[2];     // bits fixed so far, per role
  uint32_t rank[2];       // rank of the median among the values with that prefix
  float thr[2];           // fp32(3 * median) once the last pass has run
  uint32_t pad[2];
};
constexpr size_t kHistBytes = size_t(2) * 3 * kHistBins * sizeof(uint32_t);
constexpr size_t kAppendWorkspaceBytes = kHistBytes + 256;

// Decode: per (sequence, KV head) the positions are cut into n_split even
// ranges; each work-group leaves (m, l, o[128]) per query head in
// partials [B][Hkv][n_split][G][kPartStride] for the combine kernel.
constexpr int kPartStride = 132;
struct DecodePlan {
  int n_split;
  int n_pass;             // query-head passes (heads per pass: 4, 8 or 16)
  size_t partial_bytes;
};
DecodePlan make_plan(const kvq_hqmq_dims& d, int32_t batch, int32_t max_seq_len);
int heads_per_pass(int group);

float resolved_scale(const kvq_hqmq_dims& d);

// Launchers (kvq2_hqmq.hip); they return a hipError_t value (0 = success).
int launch_append(const kvq_hqmq_dims& d, const kvq_hqmq_layer& layer,
                  const kvq_hqmq_cache& cache, int32_t batch, const int32_t* start_pos,
                  const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                  const uint16_t* v_new, void* workspace, void* stream);
int launch_decode(const kvq_hqmq_dims& d, const kvq_hqmq_layer& layer,
                  const kvq_hqmq_cache& cache, int32_t batch, const int32_t* seq_len,
                  const uint16_t* q, float* out, void* workspace, const DecodePlan& plan,
                  void* stream);

}  // namespace hqmq
}  // namespace kvq
