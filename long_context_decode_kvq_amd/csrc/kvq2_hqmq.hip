// HQMQ KV-cache codec on gfx950 (include/kvq2_hqmq.h): Med3x median
// selection, encoding into paged 96-byte records, and fused split-K decode
// attention that decodes K and V inside the attention loop ("Technical
// summary: Hurwitz quaternion multiplicative quantization for KV cache
// compression", Method 1-3 and "Memory and latency").
//
// Append (one call = one Med3x batch), all launches on the caller's stream:
//   hist<0>, select<0>, hist<1>, select<1>, hist<2>, select<2>: the lower
//     median of each role's chunk norms, exactly, by a three-level radix
//     selection over the bits of the non-negative fp32 norms (LDS histograms
//     per work-group, merged with global atomics; each select pass restores
//     its histogram to zero), then thr = fp32(3 * median);
//   encode: one 32-lane half-wave per record (lane j = chunk j): norm,
//     fp16 outlier choice, fp16 r_max, radius code and the fp32 argmax over
//     the 24 S words (LDS codebook of the record's head and role), stored
//     with byte and dword stores.
//
// Decode: grid (n_split, Hkv x passes, B), 256 threads.  A token is taken by
// LPT = 32 / CPL lanes, CPL chunks each (4 channels a chunk), so a wave step
// covers 2 CPL tokens; every lane keeps q (scaled by sm_scale log2 e) and
// the value accumulators of its CPL chunks for GP query heads (four chunks
// and four heads, or one chunk and eight heads; larger groups take several
// passes of eight heads).  Per chunk: the codeword from LDS, r_hat = code r_max/255,
// logit part r_hat <q_j, c>, and after the LPT-lane sum and the lazy online
// softmax o_j += (p r_hat) c.  Each group of LPT lanes (one token slot of the
// wave step) runs its own softmax stream; the streams, the waves and the
// work-group's split are merged at the end, and a second kernel combines the
// splits.  Chunks kept in fp16 (flag bit set; their index and radius bytes
// are zero) are swapped in by selects, only in wave steps where a flag is set.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "kvq2_device.h"
#include "kvq2_hqmq_internal.h"

namespace kvq {
namespace hqmq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;       // lazy-rescale threshold (base-2 logit units)

// fp32 radius of a chunk of four values, every product and sum rounded
// separately and a correctly rounded square root.
// (HIP's __fmul_rn / __fadd_rn are plain operators that the compiler may
// fuse into an FMA, and __fsqrt_rn is the approximate hardware square root:
// contraction is switched off here and the square root is the correctly
// rounded one.)
__device__ __forceinline__ float chunk_norm(float a, float b, float c, float d) {
#pragma clang fp contract(off)
  const float s = ((a * a + b * b) + c * c) + d * d;
  return __builtin_sqrtf(s);
}

__device__ __forceinline__ float lo16(uint32_t w) { return bf16_bits_to_float(w & 0xFFFFu); }
__device__ __forceinline__ float hi16(uint32_t w) { return bf16_bits_to_float(w >> 16); }

// ------------------------------------------------------------------ append

struct AppendArgs {
  const uint16_t* x[2];            // k_new, v_new [T][Hkv][128] bf16
  const float* cb[2];              // codebooks [Hkv][24 S][4]
  uint8_t* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* start_pos;
  const int32_t* cu_new;
  int batch, total_new, n_kv_heads, page_size, n_words;
  int64_t n_chunks;                // total_new * Hkv * 32 per role
  uint32_t* hist;                  // [2 roles][3 levels][kHistBins]
  SelectState* st;
};

template <int LEVEL>
__global__ __launch_bounds__(256) void hist_kernel(AppendArgs a) {
  __shared__ uint32_t h[2][kHistBins];
  for (int i = threadIdx.x; i < 2 * kHistBins; i += 256) (&h[0][0])[i] = 0;
  uint32_t pre[2] = {0u, 0u};
  if (LEVEL > 0) {
    pre[0] = a.st->prefix[0];
    pre[1] = a.st->prefix[1];
  }
  __syncthreads();
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < a.n_chunks;
       i += int64_t(gridDim.x) * 256) {
#pragma unroll
    for (int role = 0; role < 2; ++role) {
      const uint2 w = reinterpret_cast<const uint2*>(a.x[role])[i];
      const uint32_t bits = __float_as_uint(chunk_norm(lo16(w.x), hi16(w.x), lo16(w.y), hi16(w.y)));
      if (LEVEL == 0) {
        atomicAdd(&h[role][bits >> 21], 1u);
      } else if (LEVEL == 1) {
        if ((bits >> 21) == pre[role]) atomicAdd(&h[role][(bits >> 10) & 0x7FFu], 1u);
      } else {
        if ((bits >> 10) == pre[role]) atomicAdd(&h[role][bits & 0x3FFu], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * kHistBins; i += 256) {
    const uint32_t c = (&h[0][0])[i];
    const int role = i / kHistBins, bin = i % kHistBins;
    if (c != 0) atomicAdd(&a.hist[(role * 3 + LEVEL) * kHistBins + bin], c);
  }
}

// One work-group per role: the bin holding the rank-th value of this level,
// the rank left inside it, and the histogram cleared for the next call.
template <int LEVEL>
__global__ __launch_bounds__(256) void select_kernel(AppendArgs a) {
  constexpr int kBins = LEVEL == 2 ? 1024 : kHistBins;
  constexpr int kPer = kBins / 256;
  __shared__ uint32_t sums[256];
  const int role = blockIdx.x;
  uint32_t* h = a.hist + (role * 3 + LEVEL) * kHistBins;
  const uint32_t rank = LEVEL == 0 ? uint32_t((a.n_chunks - 1) / 2) : a.st->rank[role];
  uint32_t c[kPer], s = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    c[k] = h[threadIdx.x * kPer + k];
    s += c[k];
  }
  sums[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < 256; ++i) {
      const uint32_t v = sums[i];
      sums[i] = run;
      run += v;
    }
  }
  __syncthreads();
  uint32_t before = sums[threadIdx.x];
  if (rank >= before && rank < before + s) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (rank >= before && rank < before + c[k]) {
        const uint32_t bin = threadIdx.x * kPer + k;
        const uint32_t left = rank - before;
        if (LEVEL == 0) {
          a.st->prefix[role] = bin;
        } else if (LEVEL == 1) {
          a.st->prefix[role] = (a.st->prefix[role] << 11) | bin;
        } else {
          const float med = __uint_as_float((a.st->prefix[role] << 10) | bin);
          a.st->thr[role] = 3.0f * med;
        }
        a.st->rank[role] = left;
      }
      before += c[k];
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) h[threadIdx.x * kPer + k] = 0u;
}

__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_move<kQuadXor1>(v));
  v = fmaxf(v, dpp_move<kQuadXor2>(v));
  v = fmaxf(v, dpp_move<kRowHalfMirror>(v));
  v = fmaxf(v, dpp_move<kRowMirror>(v));
  float x = v, y = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  return fmaxf(x, y);
}

// Each wave codes two records: lanes 0-31 and 32-63, lane j = chunk j.
__global__ __launch_bounds__(256) void encode_kernel(AppendArgs a) {
  __shared__ float4 cb[kMaxWords];
  const int role = blockIdx.z, h = blockIdx.y;
  {
    const float4* src = reinterpret_cast<const float4*>(a.cb[role]) + int64_t(h) * a.n_words;
    for (int i = threadIdx.x; i < a.n_words; i += 256) cb[i] = src[i];
  }
  __syncthreads();
  const float thr = a.st->thr[role];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, j = lane & 31;
  const int t = blockIdx.x * 8 + wave * 2 + half;
  const bool valid = t < a.total_new;
  const int tt = valid ? t : 0;
  // sequence of token tt: the last b with cu_new[b] <= tt
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_new[mid] <= tt) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int pos = a.start_pos[b] + (tt - a.cu_new[b]);
  const uint2 w = reinterpret_cast<const uint2*>(
      a.x[role] + (int64_t(tt) * a.n_kv_heads + h) * kHeadDim)[j];
  const float x0 = lo16(w.x), x1 = hi16(w.x), x2 = lo16(w.y), x3 = hi16(w.y);
  const float r = chunk_norm(x0, x1, x2, x3);
  const bool cand = valid && r > thr;
  const uint64_t bc = __ballot(cand);
  const uint32_t cmask = static_cast<uint32_t>(half ? (bc >> 32) : bc);
  bool keep = cand;
  if (__builtin_amdgcn_ballot_w64(__popc(cmask) > kMaxKept) != 0) {
    // rank among the candidates of the record: larger radius first, then
    // lower chunk index
    int rk = 0;
    for (int k = 0; k < 32; ++k) {
      const float rr = __shfl(r, (half << 5) + k, 64);
      const bool ck = (cmask >> k) & 1u;
      rk += (ck && (rr > r || (rr == r && k < j))) ? 1 : 0;
    }
    keep = cand && (__popc(cmask) <= kMaxKept || rk < kMaxKept);
  }
  const uint64_t bk = __ballot(keep);
  const uint32_t kmask = static_cast<uint32_t>(half ? (bk >> 32) : bk);
  const int nkeep = __popc(kmask);
  const float r_max = half_max(keep ? 0.0f : r);
  const uint32_t rmb = float_to_f16_bits(r_max);
  const float rmh = f16_bits_to_float(rmb);
  uint32_t rad = 0, idx = 0;
  if (!keep) {
    if (rmh > 0.0f) {
      const float inv = __fdiv_rn(float(kRadiusLevels), rmh);
      rad = static_cast<uint32_t>(fminf(fmaxf(rintf(r * inv), 0.0f), float(kRadiusLevels)));
    }
    if (r > 0.0f) {
#pragma clang fp contract(off)
      const float u0 = __fdiv_rn(x0, r), u1 = __fdiv_rn(x1, r);
      const float u2 = __fdiv_rn(x2, r), u3 = __fdiv_rn(x3, r);
      float best = -INFINITY;
      for (int k = 0; k < a.n_words; ++k) {
        const float4 c = cb[k];
        const float sc = ((u0 * c.x + u1 * c.y) + u2 * c.z) + u3 * c.w;
        if (sc > best) {
          best = sc;
          idx = k;
        }
      }
    }
  }
  if (!valid) return;
  const int lp = pos / a.page_size;
  if (pos < 0 || lp >= a.bt_stride) return;
  const int32_t page = a.block_table[int64_t(b) * a.bt_stride + lp];
  if (page < 0 || page >= a.num_pages) return;
  uint8_t* rec = a.pool +
                 ((int64_t(page) * a.n_kv_heads + h) * a.page_size + pos % a.page_size) *
                     kTokenBytes +
                 role * kRecordBytes;
  rec[kIdxOff + j] = static_cast<uint8_t>(idx);
  rec[kRadOff + j] = static_cast<uint8_t>(rad);
  if (j == 0) {
    *reinterpret_cast<uint32_t*>(rec + kRmaxOff) = rmb;       // r_max, then two zero bytes
    *reinterpret_cast<uint32_t*>(rec + kFlagsOff) = kmask;
  }
  if (keep) {
    const int e = __popc(kmask & ((1u << j) - 1u));
    uint2 v;
    v.x = float_to_f16_bits(x0) | (float_to_f16_bits(x1) << 16);
    v.y = float_to_f16_bits(x2) | (float_to_f16_bits(x3) << 16);
    *reinterpret_cast<uint2*>(rec + kKeptOff + 8 * e) = v;
  }
  // slots nkeep .. 2 are unused: zeroed by lanes nkeep .. 2 (whatever their
  // own chunk is; the used slots are written by the keeping lanes above)
  if (j < kMaxKept && j >= nkeep)
    *reinterpret_cast<uint2*>(rec + kKeptOff + 8 * j) = make_uint2(0u, 0u);
}

// ------------------------------------------------------------------ decode

struct DecodeArgs {
  const float* cb[2];
  const uint8_t* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t bt_stride;
  int n_q_heads, n_kv_heads, group, page_size, log2_page, n_words;
  float alpha;                     // sm_scale * log2(e)
  const int32_t* seq_len;
  const uint16_t* q;
  float* out;
  float* partials;                 // [B][Hkv][n_split][G][kPartStride]
  int n_split, n_pass;
};

// A tile is 16 consecutive positions of one (sequence, KV head): 3072
// contiguous bytes of one page (pages hold a whole number of tiles).  Each
// wave streams its tiles through a ring of kRing LDS slots with direct
// HBM -> LDS loads (three 64-lane x 16-byte loads per tile, non-temporal:
// every record is read once), so that kRing tiles are in flight per wave
// while one is decoded.
constexpr int kTileTokens = 16;
constexpr int kTileBytes = kTileTokens * kTokenBytes;
constexpr int kRing = 4;
constexpr int kDmaPerTile = kTileBytes / 1024;

// The loads and the LDS reads of the ring are written in assembly, with
// explicit waits: the compiler does not count the direct loads, so a wait
// of its own could not cover them.  Outputs of a block of several reads are
// early-clobber (no destination may share a register with an address that a
// later read of the block still uses).  M0 holds the LDS destination; lane i
// writes 16 bytes at M0 + 16 i.
__device__ __forceinline__ void dma_x4(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Sum over groups of N consecutive lanes (N = 8, 16 or 32); every lane of
// a group gets the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_move<kQuadXor1>(v);
  v += dpp_move<kQuadXor2>(v);
  v += dpp_move<kRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_move<kRowMirror>(v);
  if constexpr (N >= 32) v = xor16_sum(v);
  return v;
}

// The words of one record that a lane needs from LDS: the index and radius
// bytes of its CPL chunks, r_max (low half of hdr.x) and the flags (hdr.y).
struct RecWords {
  uint32_t idx, rad;
  uint2 hdr;
};

template <int CPL>
__device__ __forceinline__ void read_record_pair(uint32_t rec, int sub, RecWords& k,
                                                 RecWords& v) {
  const uint32_t ai = rec + CPL * sub, ah = rec + kRmaxOff;
  if constexpr (CPL == 4) {
    asm volatile(
        "ds_read_b32 %0, %6\n\t"
        "ds_read_b32 %1, %6 offset:32\n\t"
        "ds_read_b64 %2, %7\n\t"
        "ds_read_b32 %3, %6 offset:96\n\t"
        "ds_read_b32 %4, %6 offset:128\n\t"
        "ds_read_b64 %5, %7 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k.idx), "=&v"(k.rad), "=&v"(k.hdr), "=&v"(v.idx), "=&v"(v.rad), "=&v"(v.hdr)
        : "v"(ai), "v"(ah)
        : "memory");
  } else if constexpr (CPL == 2) {
    asm volatile(
        "ds_read_u16 %0, %6\n\t"
        "ds_read_u16 %1, %6 offset:32\n\t"
        "ds_read_b64 %2, %7\n\t"
        "ds_read_u16 %3, %6 offset:96\n\t"
        "ds_read_u16 %4, %6 offset:128\n\t"
        "ds_read_b64 %5, %7 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k.idx), "=&v"(k.rad), "=&v"(k.hdr), "=&v"(v.idx), "=&v"(v.rad), "=&v"(v.hdr)
        : "v"(ai), "v"(ah)
        : "memory");
  } else {
    static_assert(CPL == 1, "lane layout");
    asm volatile(
        "ds_read_u8 %0, %6\n\t"
        "ds_read_u8 %1, %6 offset:32\n\t"
        "ds_read_b64 %2, %7\n\t"
        "ds_read_u8 %3, %6 offset:96\n\t"
        "ds_read_u8 %4, %6 offset:128\n\t"
        "ds_read_b64 %5, %7 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k.idx), "=&v"(k.rad), "=&v"(k.hdr), "=&v"(v.idx), "=&v"(v.rad), "=&v"(v.hdr)
        : "v"(ai), "v"(ah)
        : "memory");
  }
}

// fp16 values of kept chunk slot e of the record at LDS address rec.
__device__ __forceinline__ float4 read_kept(uint32_t rec, int e) {
  uint2 d;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(d)
               : "v"(rec + kKeptOff + 8 * e)
               : "memory");
  return make_float4(f16_bits_to_float(d.x & 0xFFFFu), f16_bits_to_float(d.x >> 16),
                     f16_bits_to_float(d.y & 0xFFFFu), f16_bits_to_float(d.y >> 16));
}

// Chunk c of a lane's CPL chunks (chunk j = sub CPL + c): its direction or
// kept values v and its radius rh (code r_max / 255, or 1 when kept).
template <int CPL, bool KEPT>
__device__ __forceinline__ void chunk_value(const RecWords& w, uint32_t rec, const float4* cb,
                                            int sub, int c, float4& v, float& rh) {
  const uint32_t ix = (w.idx >> (8 * c)) & 0xFFu;
  const uint32_t rc = (w.rad >> (8 * c)) & 0xFFu;
  v = cb[ix];
  rh = float(rc) * (f16_bits_to_float(w.hdr.x & 0xFFFFu) * (1.0f / kRadiusLevels));
  if constexpr (KEPT) {
    const int j = sub * CPL + c;
    const uint32_t flags = w.hdr.y;
    if ((flags >> j) & 1u) {
      v = read_kept(rec, __popc(flags & ((1u << j) - 1u)));
      rh = 1.0f;
    }
  }
}

template <int CPL>
__device__ __forceinline__ uint32_t chunk_mask(int sub) {
  return ((1u << CPL) - 1u) << (sub * CPL);
}

// Logit parts of a lane's CPL key chunks: part[g] += r_hat <q_j, c>.
template <int CPL, int GP, bool KEPT>
__device__ __forceinline__ void qk_chunks(const RecWords& w, uint32_t rec, const float4* cb,
                                          int sub, const float4 (&qv)[GP][CPL],
                                          float (&part)[GP]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float4 v;
    float rh;
    chunk_value<CPL, KEPT>(w, rec, cb, sub, c, v, rh);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float d = fmaf(qv[g][c].x, v.x, fmaf(qv[g][c].y, v.y,
                           fmaf(qv[g][c].z, v.z, qv[g][c].w * v.w)));
      part[g] = fmaf(rh, d, part[g]);
    }
  }
}

// Value accumulation of a lane's CPL value chunks: acc[g][c] += (p r_hat) v.
template <int CPL, int GP, bool KEPT>
__device__ __forceinline__ void pv_chunks(const RecWords& w, uint32_t rec, const float4* cb,
                                          int sub, const float (&p)[GP],
                                          float4 (&acc)[GP][CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float4 v;
    float rh;
    chunk_value<CPL, KEPT>(w, rec, cb, sub, c, v, rh);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float wt = p[g] * rh;
      acc[g][c].x = fmaf(wt, v.x, acc[g][c].x);
      acc[g][c].y = fmaf(wt, v.y, acc[g][c].y);
      acc[g][c].z = fmaf(wt, v.z, acc[g][c].z);
      acc[g][c].w = fmaf(wt, v.w, acc[g][c].w);
    }
  }
}

template <int CPL, int GP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kernel(DecodeArgs a) {
  constexpr int LPT = 32 / CPL;          // lanes per token
  constexpr int TPS = 64 / LPT;          // tokens per pass
  constexpr int PASSES = kTileTokens / TPS;
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kRing][kTileBytes];
  __shared__ float4 cbs[2][kMaxWords];
  __shared__ float4 qs[GP][kChunks];            // q (scaled) by head and chunk
  __shared__ float kc[4][kTileTokens][GP];      // logit terms of fp16-kept key chunks
  __shared__ float wm[4][GP], wl[4][GP];
  static_assert(sizeof(ring) >= 4 * GP * kHeadDim * sizeof(float), "o' staging in the ring");
  float (*wo)[GP][kHeadDim] = reinterpret_cast<float (*)[GP][kHeadDim]>(&ring[0][0][0]);
  const int s = blockIdx.x;
  const int h = blockIdx.y / a.n_pass, pass = blockIdx.y % a.n_pass;
  const int b = blockIdx.z;
  const int G = a.group;
  const int g0 = pass * GP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int slot = lane / LPT, sub = lane % LPT;
  for (int i = threadIdx.x; i < 2 * a.n_words; i += 256) {
    const int role = i / a.n_words, k = i % a.n_words;
    cbs[role][k] = reinterpret_cast<const float4*>(a.cb[role])[int64_t(h) * a.n_words + k];
  }
  // q of this lane's chunks, scaled by alpha (heads past the group: zero)
  float4 qv[GP][CPL];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const int gq = h * G + g0 + g;
    const bool ok = g0 + g < G;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = sub * CPL + c;
      uint2 w = make_uint2(0u, 0u);
      if (ok) w = reinterpret_cast<const uint2*>(a.q + (int64_t(b) * a.n_q_heads + gq) * kHeadDim)[j];
      qv[g][c] = make_float4(lo16(w.x) * a.alpha, hi16(w.x) * a.alpha, lo16(w.y) * a.alpha,
                             hi16(w.y) * a.alpha);
      if (slot == 0) qs[g][j] = qv[g][c];
    }
  }
  // wait for q here, once: a wait of the compiler's inside the tile loop
  // would also drain the ring's loads
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      asm volatile("" : "+v"(qv[g][c].x), "+v"(qv[g][c].y), "+v"(qv[g][c].z), "+v"(qv[g][c].w));
  const int L = a.seq_len[b];
  __syncthreads();

  float m[GP], l[GP], thr[GP];
  float4 acc[GP][CPL];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    thr[g] = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[g][c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // this split's tiles [T0, T1); the wave takes tiles T0 + wave + 4 k
  const int n_tiles_all = (L + kTileTokens - 1) / kTileTokens;
  const int T0 = int(int64_t(n_tiles_all) * s / a.n_split);
  const int T1 = int(int64_t(n_tiles_all) * (s + 1) / a.n_split);
  const int my_tiles = T1 - T0 > wave ? (T1 - T0 - wave + 3) / 4 : 0;
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const_i32* bt_row = (const_i32*)(a.block_table + int64_t(b) * a.bt_stride);
  const int32_t num_pages32 = static_cast<int32_t>(min(a.num_pages, int64_t(INT32_MAX)));
  const uint32_t my_mask = chunk_mask<CPL>(sub);
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[wave][0][0]));
  // tile k of this wave (past the range, or on an invalid page: the pool's
  // first bytes, read and never used)
  auto issue = [&](int k, int r) {
    const int tile = T0 + wave + 4 * k;
    int64_t off = 0;
    if (tile < T1) {
      const int pos = tile * kTileTokens;
      const int lp = pos >> a.log2_page;
      const int32_t page = lp < a.bt_stride ? bt_row[lp] : -1;
      if (page >= 0 && page < num_pages32)
        off = ((int64_t(page) * a.n_kv_heads + h) * a.page_size + (pos & (a.page_size - 1))) *
              kTileBytes / kTileTokens;
    }
    const uint8_t* src = a.pool + off;
    const uint32_t lds = ring0 + r * kTileBytes;
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) dma_x4(src + 1024 * i, 16u * lane, lds + 1024u * i);
  };

  if (my_tiles > 0) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) issue(r, r);
    for (int k = 0; k < my_tiles; ++k) {
      const int r = k & (kRing - 1);
      // kRing tiles are outstanding: this one and the kRing - 1 after it
      wait_vmcnt<(kRing - 1) * kDmaPerTile>();
      const int pos0 = (T0 + wave + 4 * k) * kTileTokens;
      const uint32_t tile_lds = ring0 + r * kTileBytes;
      const bool partial = pos0 + kTileTokens > L;     // the sequence ends inside the tile
      // ---- the tile's fp16-kept key chunks (at most three per record; their
      // index and radius bytes are zero, so the coded path adds nothing for
      // them): lane (token tt, slot e) adds <q_j, x_e> for the e-th kept
      // chunk j of token tt, summed over e and left in kc[wave][tt][g]
      {
        const int tt = lane >> 2, e = lane & 3;
        const uint32_t krec = tile_lds + tt * kTokenBytes;
        uint32_t flags;
        asm volatile("ds_read_b32 %0, %1 offset:68\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(flags)
                     : "v"(krec)
                     : "memory");
        float cg[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) cg[g] = 0.f;
        if (pos0 + tt < L && e < __popc(flags)) {
          uint32_t f = flags;
          if (e >= 1) f &= f - 1u;
          if (e >= 2) f &= f - 1u;
          const int j = __builtin_ctz(f);
          const float4 x = read_kept(krec, e);
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            const float4 qq = qs[g][j];
            cg[g] = fmaf(qq.x, x.x, fmaf(qq.y, x.y, fmaf(qq.z, x.z, qq.w * x.w)));
          }
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          cg[g] += dpp_move<kQuadXor1>(cg[g]);
          cg[g] += dpp_move<kQuadXor2>(cg[g]);
          if (e == 0) kc[wave][tt][g] = cg[g];
        }
      }
      for (int ps = 0; ps < PASSES; ++ps) {
        const int t = ps * TPS + slot;
        const bool valid = pos0 + t < L;
        const uint32_t rec = tile_lds + t * kTokenBytes;
        RecWords wk, wv;
        read_record_pair<CPL>(rec, sub, wk, wv);
        if (partial && !valid) {
          // positions past the sequence: zero words, so that nothing of
          // their bytes reaches the sums
          wk.idx = wk.rad = wv.idx = wv.rad = 0u;
          wk.hdr = wv.hdr = make_uint2(0u, 0u);
        }
        // ---- logits: the coded chunks, then the kept chunks' terms
        float part[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) part[g] = 0.f;
        qk_chunks<CPL, GP, false>(wk, rec, cbs[0], sub, qv, part);
        float lg[GP];
        uint64_t up = 0;
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          lg[g] = group_sum<LPT>(part[g]) + kc[wave][t][g];
          lg[g] = (valid && g0 + g < G) ? lg[g] : -INFINITY;
          up |= __builtin_amdgcn_ballot_w64(lg[g] > thr[g]);
        }
        // ---- lazy online softmax, one stream per token slot
        if (up != 0) {
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            const float mn = fmaxf(m[g], lg[g]);
            if (mn > thr[g]) {
              const float corr = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - mn);
              l[g] *= corr;
#pragma unroll
              for (int c = 0; c < CPL; ++c) {
                acc[g][c].x *= corr;
                acc[g][c].y *= corr;
                acc[g][c].z *= corr;
                acc[g][c].w *= corr;
              }
              m[g] = mn;
              thr[g] = mn + kTau;
            }
          }
        }
        float p[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          p[g] = lg[g] == -INFINITY ? 0.f : exp2f(lg[g] - m[g]);
          l[g] += p[g];
        }
        // ---- values
        if (__builtin_amdgcn_ballot_w64((wv.hdr.y & my_mask) != 0u) != 0)
          pv_chunks<CPL, GP, true>(wv, rec + kRecordBytes, cbs[1], sub, p, acc);
        else
          pv_chunks<CPL, GP, false>(wv, rec + kRecordBytes, cbs[1], sub, p, acc);
      }
      // every LDS read of the slot has completed (each read block waits for
      // its data): refill it with the tile kRing steps ahead
      issue(k + kRing, r);
    }
    wait_vmcnt<0>();     // drain before the ring is reused as o' staging
  }
  __syncthreads();

  // ---- merge the TPS token-slot streams of the wave (lanes sub + LPT k)
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float M = m[g];
#pragma unroll
    for (int x = LPT; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    const float sc = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - M);
    float lt = l[g] * sc;
#pragma unroll
    for (int x = LPT; x < 64; x <<= 1) lt += __shfl_xor(lt, x, 64);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float4 o = make_float4(acc[g][c].x * sc, acc[g][c].y * sc, acc[g][c].z * sc,
                             acc[g][c].w * sc);
#pragma unroll
      for (int x = LPT; x < 64; x <<= 1) {
        o.x += __shfl_xor(o.x, x, 64);
        o.y += __shfl_xor(o.y, x, 64);
        o.z += __shfl_xor(o.z, x, 64);
        o.w += __shfl_xor(o.w, x, 64);
      }
      if (slot == 0) *reinterpret_cast<float4*>(&wo[wave][g][4 * (sub * CPL + c)]) = o;
    }
    if (lane == 0) {
      wm[wave][g] = M;
      wl[wave][g] = lt;
    }
  }
  __syncthreads();
  // ---- merge the four waves; thread (g, ch) pairs store the split partial
  float* part_base = a.partials +
                     ((int64_t(b) * a.n_kv_heads + h) * a.n_split + s) * G * kPartStride;
  for (int i = threadIdx.x; i < GP * kHeadDim; i += 256) {
    const int g = i / kHeadDim, ch = i % kHeadDim;
    if (g0 + g >= G) continue;
    float M = wm[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = (wm[w][g] == -INFINITY) ? 0.f : exp2f(wm[w][g] - M);
      lt = fmaf(sc, wl[w][g], lt);
      o = fmaf(sc, wo[w][g][ch], o);
    }
    float* dst = part_base + int64_t(g0 + g) * kPartStride;
    dst[4 + ch] = o;
    if (ch == 0) {
      dst[0] = M;
      dst[1] = lt;
    }
  }
}

// out[b][gq] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the splits
// (a sequence with no position gives a zero row).
__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  const int gq = blockIdx.x, b = blockIdx.y, ch = threadIdx.x;
  const int h = gq / a.group, g = gq % a.group;
  const float* p = a.partials + (int64_t(b) * a.n_kv_heads + h) * a.n_split * a.group * kPartStride +
                   int64_t(g) * kPartStride;
  const int64_t stride = int64_t(a.group) * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, p[s * stride]);
  float lt = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = p[s * stride];
      const float sc = ms == -INFINITY ? 0.f : exp2f(ms - M);
      lt = fmaf(sc, p[s * stride + 1], lt);
      o = fmaf(sc, p[s * stride + 4 + ch], o);
    }
  }
  a.out[(int64_t(b) * a.n_q_heads + gq) * kHeadDim + ch] = lt > 0.f ? o / lt : 0.f;
}

}  // namespace

int launch_append(const kvq_hqmq_dims& d, const kvq_hqmq_layer& layer,
                  const kvq_hqmq_cache& cache, int32_t batch, const int32_t* start_pos,
                  const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                  const uint16_t* v_new, void* workspace, void* stream) {
  AppendArgs a{};
  a.x[0] = k_new;
  a.x[1] = v_new;
  a.cb[0] = layer.codebook_K;
  a.cb[1] = layer.codebook_V;
  a.pool = cache.pool;
  a.num_pages = cache.num_pages;
  a.block_table = cache.block_table;
  a.bt_stride = cache.bt_stride;
  a.start_pos = start_pos;
  a.cu_new = cu_new;
  a.batch = batch;
  a.total_new = total_new;
  a.n_kv_heads = d.n_kv_heads;
  a.page_size = d.page_size;
  a.n_words = kPrimary * d.n_secondary;
  a.n_chunks = int64_t(total_new) * d.n_kv_heads * kChunks;
  a.hist = static_cast<uint32_t*>(workspace);
  a.st = reinterpret_cast<SelectState*>(static_cast<char*>(workspace) + kHistBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t hist_wgs = std::min<int64_t>(2048, (a.n_chunks + 255) / 256);
  const dim3 hg(static_cast<unsigned>(std::max<int64_t>(1, hist_wgs)));
  hipLaunchKernelGGL(hist_kernel<0>, hg, dim3(256), 0, st, a);
  hipLaunchKernelGGL(select_kernel<0>, dim3(2), dim3(256), 0, st, a);
  hipLaunchKernelGGL(hist_kernel<1>, hg, dim3(256), 0, st, a);
  hipLaunchKernelGGL(select_kernel<1>, dim3(2), dim3(256), 0, st, a);
  hipLaunchKernelGGL(hist_kernel<2>, hg, dim3(256), 0, st, a);
  hipLaunchKernelGGL(select_kernel<2>, dim3(2), dim3(256), 0, st, a);
  const dim3 eg((total_new + 7) / 8, d.n_kv_heads, 2);
  hipLaunchKernelGGL(encode_kernel, eg, dim3(256), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

int launch_decode(const kvq_hqmq_dims& d, const kvq_hqmq_layer& layer,
                  const kvq_hqmq_cache& cache, int32_t batch, const int32_t* seq_len,
                  const uint16_t* q, float* out, void* workspace, const DecodePlan& plan,
                  void* stream) {
  DecodeArgs a{};
  a.cb[0] = layer.codebook_K;
  a.cb[1] = layer.codebook_V;
  a.pool = cache.pool;
  a.num_pages = cache.num_pages;
  a.block_table = cache.block_table;
  a.bt_stride = cache.bt_stride;
  a.n_q_heads = d.n_q_heads;
  a.n_kv_heads = d.n_kv_heads;
  a.group = d.n_q_heads / d.n_kv_heads;
  a.page_size = d.page_size;
  a.log2_page = d.page_size == 16 ? 4 : d.page_size == 32 ? 5 : 6;
  a.n_words = kPrimary * d.n_secondary;
  a.alpha = resolved_scale(d) * kLog2e;
  a.seq_len = seq_len;
  a.q = q;
  a.out = out;
  a.partials = static_cast<float*>(workspace);
  a.n_split = plan.n_split;
  a.n_pass = plan.n_pass;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(plan.n_split, d.n_kv_heads * plan.n_pass, batch);
  if (heads_per_pass(a.group) == 4)
    hipLaunchKernelGGL((decode_kernel<4, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<1, 8>), grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(combine_kernel, dim3(d.n_q_heads, batch), dim3(128), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace hqmq
}  // namespace kvq
