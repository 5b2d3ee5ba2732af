// Quantize-append device code shared by the append kernels and the fused
// decode step (OSCAR technical summary, sec. 2.2-B: history is stored as
// INT2 after the fixed rotation and clipping; sink and recent tokens stay
// bf16).
#pragma once

#include "kvq2_device.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;

struct AppendArgs {
  const float* R[2];
  float clip[2];
  uint8_t* pool;
  int64_t num_pages;
  uint16_t* sink;
  uint16_t* recent;
  const int32_t* block_table;
  int32_t bt_stride;
  int n_kv_heads, page_size, n_sink, n_recent;
  int batch;
  const int32_t* start_pos;
  const int32_t* cu_new;
  int total_new;
  int tokens_per_block;        // multiple of kWaves
  const uint16_t* x_new[2];
  int ng;                      // (scale, zero) pairs per vector: 1, 2 or 4
  int chunk_bytes;             // 1024 + 128 ng
};

// The pinned quantizer of one value of a group with range [mn, mx]: fp16
// (scale, zero) bits and the code, each fp32 step rounded separately.
struct Quant {
  uint32_t s_bits, z_bits, code;
};
__device__ __forceinline__ Quant quantize_value(float x, float mn, float mx) {
  Quant q;
  const float s = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
  q.s_bits = float_to_f16_bits(s);
  q.z_bits = float_to_f16_bits(mn);
  const float sf = f16_bits_to_float(q.s_bits);
  const float zf = f16_bits_to_float(q.z_bits);
  q.code = 0;
  if (sf != 0.0f) {
    const float inv = __fdiv_rn(1.0f, sf);
    const float tt = __fmul_rn(__fsub_rn(x, zf), inv);
    q.code = static_cast<uint32_t>(fminf(fmaxf(rintf(tt), 0.0f), 3.0f));
  }
  return q;
}

// Quantize one rotated vector (channels lane and lane + 64) and store its
// packed codes and fp16 (scale, zero) pairs in slot t of the chunk at
// `chunk`: one pair for the vector (ng = 1), one per half of it (ng = 2:
// channel lane is in group 0, lane + 64 in group 1) or per quarter (ng = 4:
// groups lane / 32 and 2 + lane / 32).  Pinned fp32 steps, each rounded
// separately (no contraction).
__device__ void quantize_store(uint8_t* chunk, int t, int kind, float r0, float r1, float clip,
                               int lane, int ng) {
  const float x0 = fminf(fmaxf(r0, -clip), clip) + 0.0f;   // + 0 turns -0 into +0
  const float x1 = fminf(fmaxf(r1, -clip), clip) + 0.0f;
  const bool halves = ng == 4;
  float mn0 = group_min(x0, halves), mx0 = group_max(x0, halves);
  float mn1 = group_min(x1, halves), mx1 = group_max(x1, halves);
  if (ng == 1) {
    mn0 = mn1 = fminf(mn0, mn1);
    mx0 = mx1 = fmaxf(mx0, mx1);
  }
  const Quant q0 = quantize_value(x0, mn0, mx0);
  const Quant q1 = quantize_value(x1, mn1, mx1);
  const uint32_t c0 = q0.code, c1 = q1.code;
  // Four consecutive channels form a byte: channel 4g + k at bits 2k.
  uint32_t b0 = c0 << (2 * (lane & 3));
  uint32_t b1 = c1 << (2 * (lane & 3));
  b0 |= __shfl_xor(b0, 1);
  b0 |= __shfl_xor(b0, 2);
  b1 |= __shfl_xor(b1, 1);
  b1 |= __shfl_xor(b1, 2);
  if ((lane & 3) == 0) {
    const int g = lane >> 2;   // channel group of channel `lane`; group g + 16 holds lane + 64
    if (kind == 0) {
      chunk[kKCodesOff + 32 * t + g] = static_cast<uint8_t>(b0);
      chunk[kKCodesOff + 32 * t + g + 16] = static_cast<uint8_t>(b1);
    } else {
      const int base = kVCodesOff + 32 * g + 8 * (t >> 2) + (t & 3);
      chunk[base] = static_cast<uint8_t>(b0);
      chunk[base + 4] = static_cast<uint8_t>(b1);
    }
  }
  // (scale, zero) pairs: lane 0 stores its groups (and lane 32 the second
  // half's with quarters)
  if (lane == 0 || (halves && lane == 32)) {
    const int k0 = ng == 4 ? lane / 32 : 0;                 // group of channel lane
    const int k1 = ng == 4 ? 2 + lane / 32 : ng - 1;        // group of channel lane + 64
    *reinterpret_cast<uint32_t*>(chunk + param_offset(kind, t, ng, k0)) =
        q0.s_bits | (q0.z_bits << 16);
    if (ng > 1)
      *reinterpret_cast<uint32_t*>(chunk + param_offset(kind, t, ng, k1)) =
          q1.s_bits | (q1.z_bits << 16);
  }
}

// Decode-step appends (a few tokens in all): one (token, KV head, K|V)
// vector per wave, four waves per work-group sharing (KV head, K|V).  Same
// arithmetic and destinations as quantize_append_kernel; what differs is the
// order of the memory accesses, since at this size the kernel is a chain of
// dependent loads: the sequence lookup reads cu_new and start_pos with one
// vector load per lane (a ballot finds the sequence) instead of a binary
// search, and the new vector, that lookup and the R staging are all issued
// before the first wait; the ring slot and block-table reads that depend on
// the position follow as one more round.
// Block (bx, h, kind) of the grid (ceil(total_new / 4), Hkv, 2); Rs (64 KiB)
// and xs are the work-group's LDS.
__device__ __forceinline__ void append_step_block(const AppendArgs& a, int bx, int h, int kind,
                                                  float* Rs, double (*xs)[kHeadDim]) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = __builtin_amdgcn_readfirstlane(bx * kWaves + wave);
  const bool active = n < a.total_new;
  const int nn = active ? n : 0;
  // the new vector (depends on the token index only)
  const uint16_t* x = a.x_new[kind] + (int64_t(nn) * a.n_kv_heads + h) * kHeadDim;
  const uint32_t xr0 = x[lane], xr1 = x[lane + 64];
  // Sequence of token n: the first b with cu_new[b + 1] > n (cu_new is
  // non-decreasing, so the sequences that end at or before n are a prefix).
  int b = a.batch, first = 0, last = 0, start = -1;
  for (int base = 0; base < a.batch; base += 64) {
    const int i = base + lane;
    const bool in = i < a.batch;
    const int hi = in ? a.cu_new[i + 1] : INT32_MAX;
    const int lo = in ? a.cu_new[i] : 0;
    const int sp = in ? a.start_pos[i] : -1;
    const int cnt = __builtin_amdgcn_readfirstlane(
        static_cast<int>(__popcll(__builtin_amdgcn_ballot_w64(hi <= nn))));
    if (cnt < 64) {
      b = base + cnt;
      first = __builtin_amdgcn_readlane(lo, cnt);
      last = __builtin_amdgcn_readlane(hi, cnt);
      start = __builtin_amdgcn_readlane(sp, cnt);
      break;
    }
  }
  // R rows into registers; stored to LDS once the dependent reads are issued
  float4 rr[kHeadDim * kHeadDim / 4 / 256];
  {
    const float4* src = reinterpret_cast<const float4*>(a.R[kind] + int64_t(h) * kHeadDim * kHeadDim);
#pragma unroll
    for (int k = 0; k < kHeadDim * kHeadDim / 4 / 256; ++k) rr[k] = src[threadIdx.x + 256 * k];
  }
  const bool ok = active && b < a.batch && start >= 0;
  const int W = a.n_recent;
  const int ns = a.n_sink;
  const int pos = start + (n - first);
  const int end = start + (last - first);
  const int64_t seq_head = int64_t(ok ? b : 0) * a.n_kv_heads + h;
  const bool to_ring = pos >= ns && pos >= end - W;
  // the ring slot's occupant from before this append, if it leaves the window
  const int pold = pos - ((pos - start) / W + 1) * W;
  const bool evict = ok && to_ring && pold >= ns;
  float e0 = 0.f, e1 = 0.f;
  int64_t evict_off = -1;
  if (evict) {
    const uint16_t* src = a.recent + (seq_head * W + (pold - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
    e0 = bf16_bits_to_float(src[lane]);
    e1 = bf16_bits_to_float(src[lane + 64]);
    evict_off = chunk_offset_uniform(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                     a.page_size, b, h, pold, a.chunk_bytes);
  }
  int64_t int2_off = -1;
  if (ok && pos >= ns && !to_ring)
    int2_off = chunk_offset_uniform(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                    a.page_size, b, h, pos, a.chunk_bytes);
  {
    float4* dst = reinterpret_cast<float4*>(Rs);
#pragma unroll
    for (int k = 0; k < kHeadDim * kHeadDim / 4 / 256; ++k) dst[threadIdx.x + 256 * k] = rr[k];
  }
  xs[wave][lane] = double(bf16_bits_to_float(xr0));
  xs[wave][lane + 64] = double(bf16_bits_to_float(xr1));
  __syncthreads();
  if (!ok) return;
  const float clip = a.clip[kind];
  if (evict_off >= 0)
    quantize_store(a.pool + evict_off, pold % kChunkTokens, kind, e0, e1, clip, lane, a.ng);

  // Pinned rotation of the new vector.
  double acc0 = 0.0, acc1 = 0.0;
#pragma unroll 8
  for (int j = 0; j < kHeadDim; ++j) {
    const double xj = xs[wave][j];
    acc0 = __fma_rn(xj, double(Rs[j * kHeadDim + lane]), acc0);
    acc1 = __fma_rn(xj, double(Rs[j * kHeadDim + lane + 64]), acc1);
  }
  const uint32_t rb0 = float_to_bf16_bits(__double2float_rn(acc0));
  const uint32_t rb1 = float_to_bf16_bits(__double2float_rn(acc1));

  if (pos < ns) {
    uint16_t* dst = a.sink + (seq_head * ns + pos) * 2 * kHeadDim + kind * kHeadDim;
    dst[lane] = static_cast<uint16_t>(rb0);
    dst[lane + 64] = static_cast<uint16_t>(rb1);
  } else if (!to_ring) {
    if (int2_off >= 0)
      quantize_store(a.pool + int2_off, pos % kChunkTokens, kind, bf16_bits_to_float(rb0),
                     bf16_bits_to_float(rb1), clip, lane, a.ng);
  } else {
    uint16_t* dst = a.recent + (seq_head * W + (pos - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
    dst[lane] = static_cast<uint16_t>(rb0);
    dst[lane + 64] = static_cast<uint16_t>(rb1);
  }
}

// Kernel arguments of an append (the validated ABI structures).
inline AppendArgs make_append_args(const kvq_dims& d, const kvq_layer& layer, const kvq_cache& cache,
                                   int32_t batch, const int32_t* start_pos, const int32_t* cu_new,
                                   int32_t total_new, const uint16_t* k_new,
                                   const uint16_t* v_new) {
  AppendArgs a{};
  a.R[0] = layer.R_K;
  a.R[1] = layer.R_V;
  a.clip[0] = layer.clip_K;
  a.clip[1] = layer.clip_V;
  a.pool = cache.pool;
  a.num_pages = cache.num_pages;
  a.sink = cache.sink;
  a.recent = cache.recent;
  a.block_table = cache.block_table;
  a.bt_stride = cache.bt_stride;
  a.n_kv_heads = d.n_kv_heads;
  a.page_size = d.page_size;
  a.n_sink = d.n_sink;
  a.n_recent = d.n_recent;
  a.batch = batch;
  a.start_pos = start_pos;
  a.cu_new = cu_new;
  a.total_new = total_new;
  a.x_new[0] = k_new;
  a.x_new[1] = v_new;
  a.ng = kHeadDim / (d.quant_group > 0 ? d.quant_group : kHeadDim);
  a.chunk_bytes = chunk_bytes_for(a.ng);
  // Decode-step appends (a few tokens per sequence): one token per wave, for
  // parallelism; medium ones 16 per work-group; bulk appends 256, so that
  // each work-group stages R once per 256 vectors.
  a.tokens_per_block = total_new <= kStepAppendMax ? kWaves : total_new <= 8192 ? 16 : 256;
  return a;
}

}  // namespace
}  // namespace kvq
