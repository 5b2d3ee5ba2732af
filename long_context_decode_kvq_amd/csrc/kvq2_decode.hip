// Decode dispatch: fills the kernel arguments from the validated ABI
// structures, carves the caller's workspace into arrival counters and
// split-K partials, and launches the selected decode kernel.
#include <cmath>

#include "kvq2_decode_common.h"

namespace kvq {

namespace {

// Query rotation pre-pass, one work-group per (KV head, sequence):
// q'[g] = alpha * R_K[h]^T q[b][hG+g] (OSCAR summary sec. 2.2-B: the query is
// rotated once instead of un-rotating every cached key), plus sum(q'[g]) and
// the exponent e with 2^-e max|q'[g]| < 1 used to scale f16 MFMA operands.
__global__ __launch_bounds__(256) void rotate_q_kernel(DecodeArgs a) {
  __shared__ float qraw[kMaxGroup][kHeadDim];
  __shared__ float part[2][kMaxGroup][kHeadDim];
  __shared__ float qs[kMaxGroup][kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.group;
  const int tid = threadIdx.x;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    qraw[g][c] = bf16_bits_to_float(a.q[(int64_t(b) * a.n_q_heads + h * G + g) * kHeadDim + c]);
  }
  __syncthreads();
  // Thread (half, c) sums j in [64 half, 64 half + 64) for every head of the
  // group: one coalesced load of R row j feeds G independent FMA chains.
  const float* R = a.R_K + int64_t(h) * kHeadDim * kHeadDim;
  {
    const int c = tid & (kHeadDim - 1), half = tid >> 7;
    float acc[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) acc[g] = 0.0f;
    for (int j0 = 64 * half; j0 < 64 * half + 64; j0 += 16) {
      float r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) r[u] = R[(j0 + u) * kHeadDim + c];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
          if (g < G) acc[g] = fmaf(r[u], qraw[g][j0 + u], acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g)
      if (g < G) part[half][g][c] = acc[g];
  }
  __syncthreads();
  float* dst = a.qrot + (int64_t(b) * a.n_q_heads + int64_t(h) * G) * kQStride;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    const float v = (part[0][g][c] + part[1][g][c]) * a.alpha;
    qs[g][c] = v;
    dst[g * kQStride + c] = v;
  }
  __syncthreads();
  __shared__ float qsum[kMaxGroup];
  __shared__ int qexp[kMaxGroup];
  const int wave = tid >> 6, lane = tid & 63;
  for (int g = wave; g < G; g += blockDim.x / 64) {
    const float v0 = qs[g][lane], v1 = qs[g][lane + 64];
    const float sum = wave_sum(v0 + v1);
    const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    if (lane == 0) {
      const int e = mx > 0.f ? ilogbf(mx) + 1 : 0;
      dst[g * kQStride + kHeadDim] = sum;
      dst[g * kQStride + kHeadDim + 1] = float(e);
      qsum[g] = sum;
      qexp[g] = e;
    }
  }
  __syncthreads();
  // QK operand of the MFMA kernel in its per-lane layout: lane (gq, n) holds
  // column n = 2GP p + GP t + g (t = 0: f16 hi part, 1: lo part of q'[g]
  // scaled by 2^-e_g 2^(8 - 2s)) for the 32 k-slots of its lane group.
  if (a.gp == 0) return;
  const int GP = a.gp;
  uint32_t* bq = a.bq + (int64_t(b) * a.n_kv_heads + h) * kBqWords;
  {
    const int kk = tid >> 6;                 // 4 k-steps x 64 lanes
    const int gq = lane >> 4, n = lane & 15;
    const int j = n % (2 * GP), g = j % GP;
    const bool hi_col = j < GP, ok = g < G;
    const float down = ok ? ldexpf(1.0f, -qexp[g]) : 0.f;
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
      for (int e = 0; e < 2; ++e) {
        int ch, sc;
        kslot_channel(gq, kk, 2 * q + e, ch, sc);
        const float v = ok ? qs[g][ch] * down * ldexpf(1.0f, 8 - 2 * sc) : 0.f;
        const _Float16 vh = static_cast<_Float16>(v);
        const _Float16 vl = static_cast<_Float16>(v - static_cast<float>(vh));
        const uint32_t bits = __builtin_bit_cast(uint16_t, hi_col ? vh : vl);
        word |= bits << (16 * e);
      }
      bq[lane * 16 + kk * 4 + q] = word;
    }
    if (kk == 0) {
      const float qscale = ok ? ldexpf(1.0f, 16 + qexp[g]) : 1.0f;
      reinterpret_cast<float*>(bq)[64 * 16 + 2 * lane] = qscale;
      reinterpret_cast<float*>(bq)[64 * 16 + 2 * lane + 1] = ok ? qsum[g] / qscale : 0.f;
    }
  }
}

// Tile prefix of the MFMA decode (one work-group): W_b = max(1, number of
// whole INT2 tiles of sequence b), tile_prefix[b] = W_0 + ... + W_{b-1}.
// A sequence with no INT2 tile counts one (empty) tile so that a work-group
// still takes its token-by-token list.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(DecodeArgs a) {
  __shared__ int part[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  const int npt = 16 / (2 * a.gp);
  if (tid == 0) { carry = 0; a.tile_prefix[0] = 0; }
  __syncthreads();
  for (int base = 0; base < a.batch; base += 1024) {
    const int b = base + tid;
    int w = 0;
    if (b < a.batch) {
      const Int2Range rg = int2_range(a, a.seq_len[b], npt);
      w = max(1, (rg.cl - rg.cf) / npt);
    }
    part[tid] = w;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {      // inclusive scan (Hillis-Steele)
      const int v = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    if (b < a.batch) a.tile_prefix[b + 1] = carry + part[tid];
    __syncthreads();
    if (tid == 1023) carry += part[1023];
    __syncthreads();
  }
}

}  // namespace

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);
int launch_decode_mfma(const DecodeArgs& a, int batch, int max_seq_len, void* stream);

int launch_decode(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                  const kvq_cache& cache, int32_t batch, const int32_t* seq_len,
                  int32_t max_seq_len, const uint16_t* q, float* out, void* workspace,
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
  a.work_counter = a.tickets + int64_t(batch) * d.n_kv_heads;
  a.batch = batch;
  char* ws = static_cast<char*>(workspace);
  a.qrot = reinterpret_cast<float*>(ws + plan.ticket_bytes);
  a.bq = reinterpret_cast<uint32_t*>(ws + plan.ticket_bytes + plan.qrot_bytes);
  a.tile_prefix = reinterpret_cast<int32_t*>(ws + plan.ticket_bytes + plan.qrot_bytes + plan.bq_bytes);
  a.partials = reinterpret_cast<float*>(ws + plan.ticket_bytes + plan.qrot_bytes + plan.bq_bytes +
                                        plan.prefix_bytes);
  const int G = a.group;
  a.gp = (which == kDecodeValu || G > 8) ? 0 : (G <= 2 ? 2 : G <= 4 ? 4 : 8);
  a.n_split_int2 = plan.n_split_int2;
  a.n_split_big = plan.n_split_big;
  a.n_split_small = plan.n_split_small;
  a.n_split = plan.n_split;
  hipLaunchKernelGGL(rotate_q_kernel, dim3(d.n_kv_heads, batch), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  int err = static_cast<int>(hipGetLastError());
  if (err != 0) return err;
  if (which == kDecodeValu || a.gp == 0) return launch_decode_valu(a, batch, stream);
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream),
                     a);
  err = static_cast<int>(hipGetLastError());
  if (err != 0) return err;
  return launch_decode_mfma(a, batch, max_seq_len, stream);
}

}  // namespace kvq
