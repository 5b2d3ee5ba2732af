// Device helpers shared by the libkvq2 HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq2_internal.h"

namespace kvq {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

__device__ __forceinline__ uint32_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Cross-lane moves within 16-lane rows (DPP): QUAD_XOR1/2 exchange lanes
// i ^ 1 and i ^ 2; ROW_HALF_MIRROR maps lane i of 8 to 7 - i and ROW_MIRROR
// lane i of 16 to 15 - i.  After the two quad steps every lane of a quad
// holds the quad's value, so the mirrors then act as butterflies over quads
// and half rows.
enum : int { kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, true));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Reductions over all 64 lanes of a wave (every lane must be active): four
// DPP butterfly steps give each 16-lane row its total, the four row totals
// are combined through scalar registers, so every lane gets the same value.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<kQuadXor1>(v));
  v = fmaxf(v, dpp_move<kQuadXor2>(v));
  v = fmaxf(v, dpp_move<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_move<kRowMirror>(v));
  return fmaxf(fmaxf(read_lane(v, 0), read_lane(v, 16)), fmaxf(read_lane(v, 32), read_lane(v, 48)));
}

__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_move<kQuadXor1>(v));
  v = fminf(v, dpp_move<kQuadXor2>(v));
  v = fminf(v, dpp_move<kRowHalfMirror>(v));
  v = fminf(v, dpp_move<kRowMirror>(v));
  return fminf(fminf(read_lane(v, 0), read_lane(v, 16)), fminf(read_lane(v, 32), read_lane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<kQuadXor1>(v);
  v += dpp_move<kQuadXor2>(v);
  v += dpp_move<kRowHalfMirror>(v);
  v += dpp_move<kRowMirror>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Butterfly sums across 16-lane rows (gfx950 row swaps): v_permlane16_swap
// exchanges the odd rows of its first operand with the even rows of its
// second, v_permlane32_swap the upper half of the first with the lower half
// of the second.  With both operands equal to v the two registers then hold
// v[i] and v[i ^ 16] (v[i ^ 32]) in row order, so both lanes of a pair add
// them in the same order.  Written in assembly: the compiler's builtin
// folded the two results of such a swap into one.  The s_nop covers the
// wait states between the VALU writes of the operands and the swap.
__device__ __forceinline__ float xor16_sum(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

__device__ __forceinline__ float xor32_sum(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

// Device-coherent global accesses for data handed between work-groups of one
// launch (the VALU decode's split partials and arrival tickets).  The XCDs of
// the GPU have separate L2 caches; agent-scope atomic loads and stores are
// coherent across them.  The hand-off follows the HIP memory model: the
// writer stores its partial with agent-scope atomic stores and takes the
// arrival ticket with an agent-scope acquire-release read-modify-write; the
// last arriver's ticket operation is then an acquire of every earlier
// writer's release, and it reads the partials with agent-scope loads after a
// work-group barrier.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Arrival ticket: releases this wave's earlier stores, acquires those of the
// waves that took the ticket before.
__device__ __forceinline__ int fetch_add_acq_rel_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// Min / max over the lanes of one quantization group: the whole wave, or
// (halves) each half of it (lanes 0-31 and 32-63).  All 64 lanes active.
__device__ __forceinline__ float group_min(float v, bool halves) {
  v = fminf(v, dpp_move<kQuadXor1>(v));
  v = fminf(v, dpp_move<kQuadXor2>(v));
  v = fminf(v, dpp_move<kRowHalfMirror>(v));
  v = fminf(v, dpp_move<kRowMirror>(v));
  const float lo = fminf(read_lane(v, 0), read_lane(v, 16));
  const float hi = fminf(read_lane(v, 32), read_lane(v, 48));
  return halves ? ((threadIdx.x & 32) ? hi : lo) : fminf(lo, hi);
}

__device__ __forceinline__ float group_max(float v, bool halves) {
  v = fmaxf(v, dpp_move<kQuadXor1>(v));
  v = fmaxf(v, dpp_move<kQuadXor2>(v));
  v = fmaxf(v, dpp_move<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_move<kRowMirror>(v));
  const float lo = fmaxf(read_lane(v, 0), read_lane(v, 16));
  const float hi = fmaxf(read_lane(v, 32), read_lane(v, 48));
  return halves ? ((threadIdx.x & 32) ? hi : lo) : fmaxf(lo, hi);
}

// Byte offset of (scale, zero) of quantization group k of slot t in a chunk
// with ng groups per vector (kind 0 = K, 1 = V).
__device__ __forceinline__ int param_offset(int kind, int t, int ng, int k) {
  return 1024 + kind * 64 * ng + 4 * (t * ng + k);
}

// Byte offset of the chunk (chunk_bytes long) holding position `pos` of
// sequence b, KV head h; -1 if the block-table entry is outside
// [0, num_pages).
__device__ __forceinline__ int64_t chunk_offset(const int32_t* block_table, int32_t bt_stride,
                                                int64_t num_pages, int n_kv_heads, int page_size,
                                                int b, int h, int pos, int chunk_bytes) {
  if (pos < 0) return -1;
  const int lp = pos / page_size;
  if (lp >= bt_stride) return -1;
  const int32_t page = block_table[int64_t(b) * bt_stride + lp];
  if (page < 0 || page >= num_pages) return -1;
  const int cpp = page_size / kChunkTokens;
  return ((int64_t(page) * n_kv_heads + h) * cpp + (pos % page_size) / kChunkTokens) *
         int64_t(chunk_bytes);
}

// Same, for a wave-uniform position: the block-table entry is read through the
// scalar data cache (the table is read-only while a kernel runs).
__device__ __forceinline__ int64_t chunk_offset_uniform(const int32_t* block_table,
                                                        int32_t bt_stride, int64_t num_pages,
                                                        int n_kv_heads, int page_size, int b,
                                                        int h, int pos, int chunk_bytes) {
  pos = __builtin_amdgcn_readfirstlane(pos);
  if (pos < 0) return -1;
  const int lp = pos / page_size;
  if (lp >= bt_stride) return -1;
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const int32_t page = ((const_i32*)block_table)[int64_t(b) * bt_stride + lp];
  if (page < 0 || page >= num_pages) return -1;
  const int cpp = page_size / kChunkTokens;
  return ((int64_t(page) * n_kv_heads + h) * cpp + (pos % page_size) / kChunkTokens) *
         int64_t(chunk_bytes);
}

}  // namespace kvq
