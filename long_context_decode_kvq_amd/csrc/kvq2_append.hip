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
#include "kvq2_append_common.h"

namespace kvq {
namespace {

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
                                         a.page_size, b, h, pold, a.chunk_bytes);
        if (off >= 0)
          quantize_store(a.pool + off, pold % kChunkTokens, kind, r0, r1, clip, lane, a.ng);
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
                                       a.page_size, b, h, pos, a.chunk_bytes);
      if (off >= 0)
        quantize_store(a.pool + off, pos % kChunkTokens, kind, bf16_bits_to_float(rb0),
                       bf16_bits_to_float(rb1), clip, lane, a.ng);
    } else {
      uint16_t* dst = a.recent + (seq_head * W + (pos - ns) % W) * 2 * kHeadDim + kind * kHeadDim;
      dst[lane] = static_cast<uint16_t>(rb0);
      dst[lane + 64] = static_cast<uint16_t>(rb1);
    }
  }
}

__global__ __launch_bounds__(256) void append_step_kernel(AppendArgs a) {
  __shared__ float Rs[kHeadDim * kHeadDim];
  __shared__ double xs[kWaves][kHeadDim];
  append_step_block(a, blockIdx.x, blockIdx.y, blockIdx.z, Rs, xs);
}

}  // namespace

int launch_quantize_append(const kvq_dims& d, float /*sm_scale*/, const kvq_layer& layer,
                           const kvq_cache& cache, int32_t batch, const int32_t* start_pos,
                           const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                           const uint16_t* v_new, void* stream) {
  AppendArgs a = make_append_args(d, layer, cache, batch, start_pos, cu_new, total_new, k_new,
                                  v_new);
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
