// Quantize-append kernel (OSCAR technical summary, sec. 2.2-B: history is
// stored as INT2 after the fixed rotation and clipping; sink and recent
// tokens stay bf16).
//
// One wave (64 lanes) handles one new (token, KV head, K|V) head-vector;
// lane l owns channels l and l + 64.  A work-group of four waves shares one
// (KV head, K|V) pair and stages that 64 KiB rotation matrix in LDS once for
// the tokens it handles (16 for decode-size appends, 256 for bulk appends).
//
// Per vector:
//   1. If the token is written to the recent ring and the slot's previous
//      occupant (an older token of this sequence) leaves the window, that
//      occupant is quantized from its stored bf16 values into its INT2 page
//      first.  The same lanes read the slot before they overwrite it.
//   2. r = bf16(fp32(R^T x)) with fp64 accumulation in channel order.
//   3. Sink slot, INT2 page (quantize + pack), or ring slot, by position.
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
};

// Quantize one rotated vector (channels lane and lane + 64) and store its
// packed codes and fp16 (scale, zero) in slot t of the chunk at `chunk`.
// Pinned fp32 steps, each rounded separately (no contraction).
__device__ void quantize_store(uint8_t* chunk, int t, int kind, float r0, float r1, float clip,
                               int lane) {
  const float x0 = fminf(fmaxf(r0, -clip), clip) + 0.0f;   // + 0 turns -0 into +0
  const float x1 = fminf(fmaxf(r1, -clip), clip) + 0.0f;
  const float mn = wave_min(fminf(x0, x1));
  const float mx = wave_max(fmaxf(x0, x1));
  const float s = __fdiv_rn(__fsub_rn(mx, mn), 3.0f);
  const uint32_t s_bits = float_to_f16_bits(s);
  const uint32_t z_bits = float_to_f16_bits(mn);
  const float sf = f16_bits_to_float(s_bits);
  const float zf = f16_bits_to_float(z_bits);
  uint32_t c0 = 0, c1 = 0;
  if (sf != 0.0f) {
    const float inv = __fdiv_rn(1.0f, sf);
    const float t0 = __fmul_rn(__fsub_rn(x0, zf), inv);
    const float t1 = __fmul_rn(__fsub_rn(x1, zf), inv);
    c0 = static_cast<uint32_t>(fminf(fmaxf(rintf(t0), 0.0f), 3.0f));
    c1 = static_cast<uint32_t>(fminf(fmaxf(rintf(t1), 0.0f), 3.0f));
  }
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
  if (lane == 0) {
    const int off = (kind == 0 ? kKParamsOff : kVParamsOff) + 4 * t;
    *reinterpret_cast<uint32_t*>(chunk + off) = s_bits | (z_bits << 16);
  }
}

__global__ __launch_bounds__(256) void quantize_append_kernel(AppendArgs a) {
  __shared__ float Rs[kHeadDim * kHeadDim];
  __shared__ double xs[kWaves][kHeadDim];
  const int h = blockIdx.y;
  const int kind = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  {
    const float4* src = reinterpret_cast<const float4*>(a.R[kind] + int64_t(h) * kHeadDim * kHeadDim);
    float4* dst = reinterpret_cast<float4*>(Rs);
    for (int i = threadIdx.x; i < kHeadDim * kHeadDim / 4; i += blockDim.x) dst[i] = src[i];
  }
  __syncthreads();
  const float clip = a.clip[kind];
  const int W = a.n_recent;
  const int ns = a.n_sink;
  const int per_wave = a.tokens_per_block / kWaves;
  // The token index is wave-uniform: the sequence lookup reads cu_new and
  // start_pos through the scalar cache (a chain of vector loads would be the
  // latency of a decode-step append).
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const_i32* cu_new = (const_i32*)a.cu_new;
  const_i32* start_pos = (const_i32*)a.start_pos;
  for (int it = 0; it < per_wave; ++it) {
    const int n = __builtin_amdgcn_readfirstlane(blockIdx.x * a.tokens_per_block + wave * per_wave + it);
    if (n >= a.total_new) break;
    // Sequence of token n: the largest b with cu_new[b] <= n.
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_new[mid] <= n) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int start = start_pos[b];
    if (start < 0) continue;   // invalid length: nothing is written
    const int pos = start + (n - cu_new[b]);
    const int end = start + (cu_new[b + 1] - cu_new[b]);
    const int64_t seq_head = int64_t(b) * a.n_kv_heads + h;
    const bool to_ring = pos >= ns && pos >= end - W;

    if (to_ring) {
      // The ring slot's occupant from before this append, if it leaves the window.
      const int pold = pos - ((pos - start) / W + 1) * W;
      if (pold >= ns) {
        const uint16_t* src = a.recent + (seq_head * W + (pold - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
        const float r0 = bf16_bits_to_float(src[lane]);
        const float r1 = bf16_bits_to_float(src[lane + 64]);
        const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                         a.page_size, b, h, pold);
        if (off >= 0) quantize_store(a.pool + off, pold % kChunkTokens, kind, r0, r1, clip, lane);
      }
    }

    // Pinned rotation of the new vector.
    const uint16_t* x = a.x_new[kind] + (int64_t(n) * a.n_kv_heads + h) * kHeadDim;
    xs[wave][lane] = double(bf16_bits_to_float(x[lane]));
    xs[wave][lane + 64] = double(bf16_bits_to_float(x[lane + 64]));
    __builtin_amdgcn_wave_barrier();
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll 8
    for (int j = 0; j < kHeadDim; ++j) {
      const double xj = xs[wave][j];
      acc0 = __fma_rn(xj, double(Rs[j * kHeadDim + lane]), acc0);
      acc1 = __fma_rn(xj, double(Rs[j * kHeadDim + lane + 64]), acc1);
    }
    __builtin_amdgcn_wave_barrier();
    const uint32_t rb0 = float_to_bf16_bits(__double2float_rn(acc0));
    const uint32_t rb1 = float_to_bf16_bits(__double2float_rn(acc1));

    if (pos < ns) {
      uint16_t* dst = a.sink + (seq_head * ns + pos) * 2 * kHeadDim + kind * kHeadDim;
      dst[lane] = static_cast<uint16_t>(rb0);
      dst[lane + 64] = static_cast<uint16_t>(rb1);
    } else if (!to_ring) {
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, pos);
      if (off >= 0)
        quantize_store(a.pool + off, pos % kChunkTokens, kind, bf16_bits_to_float(rb0),
                       bf16_bits_to_float(rb1), clip, lane);
    } else {
      uint16_t* dst = a.recent + (seq_head * W + (pos - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
      dst[lane] = static_cast<uint16_t>(rb0);
      dst[lane + 64] = static_cast<uint16_t>(rb1);
    }
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
__global__ __launch_bounds__(256) void append_step_kernel(AppendArgs a) {
  __shared__ float Rs[kHeadDim * kHeadDim];
  __shared__ double xs[kWaves][kHeadDim];
  const int h = blockIdx.y;
  const int kind = blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wave);
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
                                     a.page_size, b, h, pold);
  }
  int64_t int2_off = -1;
  if (ok && pos >= ns && !to_ring)
    int2_off = chunk_offset_uniform(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                    a.page_size, b, h, pos);
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
  if (evict_off >= 0) quantize_store(a.pool + evict_off, pold % kChunkTokens, kind, e0, e1, clip, lane);

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
                     bf16_bits_to_float(rb1), clip, lane);
  } else {
    uint16_t* dst = a.recent + (seq_head * W + (pos - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
    dst[lane] = static_cast<uint16_t>(rb0);
    dst[lane + 64] = static_cast<uint16_t>(rb1);
  }
}

}  // namespace

int launch_quantize_append(const kvq_dims& d, float /*sm_scale*/, const kvq_layer& layer,
                           const kvq_cache& cache, int32_t batch, const int32_t* start_pos,
                           const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                           const uint16_t* v_new, void* stream) {
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
  // Decode-step appends (a few tokens per sequence): one token per wave, for
  // parallelism; medium ones 16 per work-group; bulk appends 256, so that
  // each work-group stages R once per 256 vectors.
  a.tokens_per_block = total_new <= 1024 ? kWaves : total_new <= 8192 ? 16 : 256;
  dim3 grid((total_new + a.tokens_per_block - 1) / a.tokens_per_block, d.n_kv_heads, 2);
  if (a.tokens_per_block == kWaves)
    hipLaunchKernelGGL(append_step_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(quantize_append_kernel, grid, dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

const char* hip_error_name(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace kvq
