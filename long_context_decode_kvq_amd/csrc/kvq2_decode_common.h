// Pieces shared by the decode kernels: the query-rotation prologue, the
// work-group merge of per-wave softmax states, the split-K partial store and
// the last-arrival combine with the output inverse rotation.
//
// OSCAR technical summary, sec. 2.2-B: the fused kernel undoes the rotation;
// here that is done exactly once per query head on each side: q' = R_K^T q
// before the token loop and o = R_V o' after the split-K combine.
#pragma once

#include "kvq2_device.h"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const float* R_K;
  const float* R_V;
  const uint8_t* pool;
  int64_t num_pages;
  const uint16_t* sink;
  const uint16_t* recent;
  const int32_t* block_table;
  int32_t bt_stride;
  int n_q_heads, n_kv_heads, group, page_size, n_sink, n_recent;
  float alpha;                 // sm_scale * log2(e): logits are kept in base-2 units
  const int32_t* seq_len;
  const uint16_t* q;
  float* out;
  int32_t* tickets;            // [B * Hkv]
  float* partials;             // [B][Hkv][n_split][G][kPartialStride]
  int n_split_int2;
  int n_split;
};

// Chunk range [c_begin, c_end) of INT2 split `s` for a sequence of length L.
__device__ __forceinline__ void int2_chunk_range(const DecodeArgs& a, int L, int s, int& c_begin,
                                                 int& c_end, int& int2_end) {
  int2_end = max(a.n_sink, L - a.n_recent);
  const int first = a.n_sink / kChunkTokens;
  const int last = (int2_end + kChunkTokens - 1) / kChunkTokens;
  const int n = int2_end > a.n_sink ? last - first : 0;
  const int per = (n + a.n_split_int2 - 1) / a.n_split_int2;
  c_begin = first + min(n, s * per);
  c_end = first + min(n, (s + 1) * per);
}

// q'[g][i] = alpha * sum_j R_K[h][j][i] q[b][hG+g][j] into LDS, plus
// qsum[g] = sum_i q'[g][i].  All 256 threads take part; ends with a barrier.
template <int GP>
__device__ void rotate_queries(const DecodeArgs& a, int b, int h, float (*qraw)[kHeadDim],
                               float (*qs)[kHeadDim], float* qsum) {
  const int G = a.group;
  const int tid = threadIdx.x;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    qraw[g][c] = bf16_bits_to_float(a.q[(int64_t(b) * a.n_q_heads + h * G + g) * kHeadDim + c]);
  }
  __syncthreads();
  const float* R = a.R_K + int64_t(h) * kHeadDim * kHeadDim;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float acc = 0.0f;
#pragma unroll 8
    for (int j = 0; j < kHeadDim; ++j) acc = fmaf(R[j * kHeadDim + c], qraw[g][j], acc);
    qs[g][c] = acc * a.alpha;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int g = wave; g < G; g += blockDim.x / 64) {
    const float v = wave_sum(qs[g][lane] + qs[g][lane + 64]);
    if (lane == 0) qsum[g] = v;
  }
  __syncthreads();
}

// Merge the softmax states of the 4 waves of a work-group (m, l per head and
// unnormalized o'[128] per head, staged in LDS) and store the work-group's
// partial for split `s`.  Then take an arrival ticket; the last work-group of
// (b, h) combines all splits, applies o = R_V o' and writes `out`.
template <int GP>
__device__ void finish_work_group(const DecodeArgs& a, int b, int h, int s,
                                  float (*wm)[GP], float (*wl)[GP], float (*wo)[GP][kHeadDim],
                                  float (*ocomb)[kHeadDim]) {
  const int G = a.group;
  const int tid = threadIdx.x;
  const int64_t head = int64_t(b) * a.n_kv_heads + h;
  float* part = a.partials + (head * a.n_split + s) * G * kPartialStride;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(wm[w][g] - M);
        o += f * wo[w][g][c];
        l += f * wl[w][g];
      }
    }
    part[g * kPartialStride + 4 + c] = o;
    if (c == 0) {
      part[g * kPartialStride + 0] = M;
      part[g * kPartialStride + 1] = l;
    }
  }
  // Release: every thread makes its partial writes visible device-wide
  // before the work-group's arrival is counted.
  __threadfence();
  __syncthreads();
  __shared__ int is_last;
  if (tid == 0) {
    const int prev = atomicAdd(&a.tickets[head], 1);
    is_last = (prev == a.n_split - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();   // acquire: see every other work-group's partials

  const float* base = a.partials + head * a.n_split * G * kPartialStride;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
    for (int t = 0; t < a.n_split; ++t) M = fmaxf(M, base[(t * G + g) * kPartialStride]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
      for (int t = 0; t < a.n_split; ++t) {
        const float* p = base + (t * G + g) * kPartialStride;
        const float f = exp2f(p[0] - M);
        num += f * p[4 + c];
        den += f * p[1];
      }
    }
    ocomb[g][c] = den > 0.0f ? num / den : 0.0f;
  }
  __syncthreads();
  // o = R_V o' (row-major R_V: o_i = sum_j R_V[i][j] o'_j)
  const float* R = a.R_V + int64_t(h) * kHeadDim * kHeadDim;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    const float4* row = reinterpret_cast<const float4*>(R + c * kHeadDim);
    float acc = 0.0f;
#pragma unroll 4
    for (int j = 0; j < kHeadDim / 4; ++j) {
      const float4 r = row[j];
      acc = fmaf(r.x, ocomb[g][4 * j + 0], acc);
      acc = fmaf(r.y, ocomb[g][4 * j + 1], acc);
      acc = fmaf(r.z, ocomb[g][4 * j + 2], acc);
      acc = fmaf(r.w, ocomb[g][4 * j + 3], acc);
    }
    a.out[(int64_t(b) * a.n_q_heads + h * G + g) * kHeadDim + c] = acc;
  }
  if (tid == 0) a.tickets[head] = 0;   // ready for the next call on this workspace
}

}  // namespace kvq
