// Read-bandwidth probes (include/kvq2_probe.h): the ceilings that plain
// reads reach on the GPU the decode runs on, one for a sequential pass and
// one for the decode's own access pattern (1152-byte INT2 chunks scattered
// over the pool, read through the same non-temporal global->LDS loads with
// four tiles of two chunks in flight per wave, as the decode's stream does
// for head groups of up to four).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq2.h"
#include "kvq2_probe.h"

namespace kvq {
namespace {

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m));
  return v;
}

// One contiguous block per work-group, eight 4 KiB steps in flight, with
// non-temporal loads (the fastest of the sequential variants measured:
// grid-stride or cached loads reach 5.2-6.2 TB/s, this ~6.7-6.8 TB/s).
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* src, uint64_t n16,
                                                          uint32_t* sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t b0 = per * blockIdx.x, b1 = min(n16, b0 + per);
  uint32_t acc = 0;
  constexpr int kInFlight = 8;
  uint64_t i = b0 + threadIdx.x;
  for (; i + (kInFlight - 1) * 256 < b1; i += kInFlight * 256) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(s + i + k * 256);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < b1; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(s + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc = wave_xor(acc);
  if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x], acc);
}

// 16 bytes per lane from sbase + voff into LDS at M0 + 16 lane.
__device__ __forceinline__ void dma_x4(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}

// 4 bytes per lane from a per-lane address into LDS at M0 + 4 lane.
__device__ __forceinline__ void dma_x1(const uint8_t* vaddr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off nt"
      :
      : "v"(vaddr), "s"(lds)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

constexpr int kRing = 4;                  // tiles in flight per wave
constexpr int kTileBytes = 2 * 1024 + 256;   // two chunks' codes + both chunks' params
constexpr int kDmaPerTile = 3;

__global__ __launch_bounds__(256, 4) void chunk_read_kernel(const uint8_t* pool,
                                                            const int64_t* chunk_off,
                                                            int64_t n_chunks, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][4][kTileBytes];
  typedef const int64_t __attribute__((address_space(4))) const_i64;
  const_i64* offs = (const_i64*)chunk_off;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t n_tiles = (n_chunks + 1) / 2;
  const int64_t waves = int64_t(gridDim.x) * 4;
  const int64_t gw = int64_t(blockIdx.x) * 4 + wave;
  const int64_t t0 = n_tiles * gw / waves, t1 = n_tiles * (gw + 1) / waves;
  const int n = static_cast<int>(t1 - t0);
  uint32_t acc = 0;
  if (n > 0) {
    // Tiles past the wave's slice re-read its last tile, so that every step
    // keeps kRing tiles of loads outstanding and the wait below is exact.
    auto issue = [&](int64_t t, int k) {
      const int64_t tt = t < t1 ? t : t1 - 1;
      const int64_t c0 = 2 * tt, c1 = 2 * tt + 1 < n_chunks ? 2 * tt + 1 : 2 * tt;
      const int64_t o0 = offs[c0], o1 = offs[c1];
      const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[k][wave][0]));
      dma_x4(pool + o0, 16u * lane, lds);
      dma_x4(pool + o1, 16u * lane, lds + 1024u);
      const int64_t o = lane >= 32 ? o1 : o0;
      dma_x1(pool + o + 1024 + 4 * (lane & 31), lds + 2048u);
    };
#pragma unroll
    for (int k = 0; k < kRing; ++k) issue(t0 + k, k);
    for (int i = 0; i < n; i += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        if (i + k < n) {
          wait_vmcnt<(kRing - 1) * kDmaPerTile>();
          // one dword of each part of the slot: codes of both chunks (16 lane
          // and 1024 + 16 lane < 2048) and the params (2048 + 4 lane < 2304)
          const uint32_t base =
              static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[k][wave][0]));
          const uint32_t a_code = base + 16u * lane, a_par = base + 2048u + 4u * lane;
          uint32_t w0, w1, w2;
          asm volatile(
              "ds_read_b32 %0, %3\n\t"
              "ds_read_b32 %1, %3 offset:1024\n\t"
              "ds_read_b32 %2, %4\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(w0), "=&v"(w1), "=&v"(w2)
              : "v"(a_code), "v"(a_par)
              : "memory");
          acc ^= w0 ^ w1 ^ w2;
          issue(t0 + i + k + kRing, k);
        }
      }
    }
    wait_vmcnt<0>();
  }
  acc = wave_xor(acc);
  if (lane == 0) atomicXor(&sink[blockIdx.x], acc);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t work_groups,
                          void* stream) {
  using namespace kvq;
  if (src == nullptr || sink == nullptr || !aligned16(src) || bytes == 0 || bytes % 16 != 0 ||
      work_groups < 1 || work_groups > 65536)
    return KVQ_ERR_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3(work_groups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     static_cast<uint64_t>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kvq_probe_chunk_read(const uint8_t* pool, const int64_t* chunk_off, int64_t n_chunks,
                         uint32_t* sink, int32_t work_groups, void* stream) {
  using namespace kvq;
  if (pool == nullptr || chunk_off == nullptr || sink == nullptr || !aligned16(pool) ||
      !aligned16(chunk_off) || n_chunks < 1 || work_groups < 1 || work_groups > 65536)
    return KVQ_ERR_ARG;
  hipLaunchKernelGGL(chunk_read_kernel, dim3(work_groups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), pool, chunk_off, n_chunks, sink);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // extern "C"
