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
constexpr int kCombineSlice = 64;   // splits staged per combine pass

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
  float sigma_v;               // power of two with sigma_v * s_V <= 1 for every V scale
  int log2_sigma_v;            // log2(sigma_v)
  int log2_cpp;                // log2(page_size / 16)
  int64_t page_bytes;          // bytes of one physical page: Hkv * page_size / 16 * 1152
  const int32_t* seq_len;
  const uint16_t* q;
  float* out;
  int32_t* tickets;            // [B * Hkv]
  int32_t* work_counter;       // [2]: next work item, work-groups finished
  int batch;
  float* qrot;                 // [B][Hq][kQStride]: alpha R_K^T q, its sum, f16 exponent
  uint32_t* bq;                // [B * Hkv][kBqWords]: QK MFMA operand and lane constants
  int gp;                      // MFMA head-group width (2, 4 or 8)
  float* partials;             // [B][Hkv][n_split][G][kPartialStride]
  int n_split_int2;            // INT2 splits per (b, h) = n_split_big + n_split_small
  int n_split_big;             // splits over the first 3/4 of the tiles (scheduled first)
  int n_split_small;           // splits over the last 1/4 (scheduled after every big one)
  int n_split;
  // MFMA decode: tile_prefix[b] = sum over b' < b of max(1, INT2 tiles of
  // sequence b') (B + 1 entries, written by a pre-pass); the launch cuts the
  // concatenated tiles of all (b, h) into equal ranges, one per work-group.
  int32_t* tile_prefix;
};

// INT2 work of a sequence of length L is split in two parts:
//  * whole tiles of `npt` fully valid 16-token chunks [cf, cl), cut into
//    n_split_int2 contiguous tile ranges (one per split work-group);
//  * the few INT2 positions outside them (the partial chunk after the sink,
//    the partial chunk before the recent window and a sub-tile remainder),
//    which the work-group of the bf16 segments handles token by token.
struct Int2Range {
  int int2_end;   // INT2 positions are [n_sink, int2_end)
  int cf, cl;     // tiled chunks [cf, cl), cl - cf a multiple of npt
};

__device__ __forceinline__ Int2Range int2_range(const DecodeArgs& a, int L, int npt) {
  Int2Range r;
  r.int2_end = max(a.n_sink, L - a.n_recent);
  r.cf = (a.n_sink + kChunkTokens - 1) / kChunkTokens;
  const int full_end = r.int2_end / kChunkTokens;
  r.cl = full_end > r.cf ? r.cf + npt * ((full_end - r.cf) / npt) : r.cf;
  return r;
}

// Tile range [t_begin, t_end) of INT2 split s.  Splits s < n_split_big
// share the first 3/4 of the n tiles evenly, the n_split_small others the
// rest: the work queue hands out every big split before any small one, so
// the launch ends on short items (with n_split_small = 0, one even split).
__device__ __forceinline__ void split_tiles(const DecodeArgs& a, const Int2Range& r, int npt, int s,
                                            int& t_begin, int& t_end) {
  const int n = (r.cl - r.cf) / npt;
  const int nb = a.n_split_big, nsm = a.n_split_small;
  const int n_big = nsm > 0 ? (3 * n) / 4 : n;   // tiles of the big splits
  if (s < nb) {
    t_begin = int(int64_t(n_big) * s / nb);
    t_end = int(int64_t(n_big) * (s + 1) / nb);
  } else {
    const int j = s - nb;
    t_begin = n_big + int(int64_t(n - n_big) * j / nsm);
    t_end = n_big + int(int64_t(n - n_big) * (j + 1) / nsm);
  }
}

// QK k-slot -> channel map of the MFMA decode kernel: k-slot i (pair q = i/2,
// element e = i%2) of k-step kk for lane group gq holds channel
// 32gq + 16(kk/2) + local, where the code was extracted at scale 2^(2s - 24)
// (one AND per f16 pair, see the MFMA kernel).
__device__ __forceinline__ void kslot_channel(int gq, int kk, int i, int& ch, int& s) {
  const int q = i >> 1, e = i & 1;
  const int local = (kk & 1) ? (4 + q + 8 * e) : (q + 8 * e);
  ch = 32 * gq + 16 * (kk >> 1) + local;
  s = (kk & 1) ? (q == 0 ? 4 : q) : q;
}

// The rotated queries of (b, h), computed once per call by the rotation
// pre-pass, into LDS: q'[g][:] (alpha folded in), qsum[g] = sum_i q'[g][i]
// and qexp[g] with 2^-qexp[g] max|q'[g]| < 1.  Ends with a barrier.
template <int GP>
__device__ void load_queries(const DecodeArgs& a, int b, int h, float (*qs)[kHeadDim],
                             float* qsum, int* qexp) {
  const int G = a.group;
  const float* src = a.qrot + (int64_t(b) * a.n_q_heads + int64_t(h) * G) * kQStride;
  for (int i = threadIdx.x; i < G * kHeadDim; i += blockDim.x)
    qs[i / kHeadDim][i % kHeadDim] = src[(i / kHeadDim) * kQStride + i % kHeadDim];
  if (threadIdx.x < G) {
    qsum[threadIdx.x] = src[threadIdx.x * kQStride + kHeadDim];
    qexp[threadIdx.x] = static_cast<int>(src[threadIdx.x * kQStride + kHeadDim + 1]);
  }
  __syncthreads();
}

// Online-softmax update of one 16-token tile for a wave whose lane (t, qq)
// = (lane / 4, lane % 4) holds the logit of token t in lg[g] (-inf when
// masked; the four lanes of a token hold the same value).  Updates the
// running (m, l) per head, returns the correction factor per head and
// leaves p = exp2(logit - m) in lg.
template <int GP>
__device__ __forceinline__ void softmax_tile16(int G, int qq, float* lg, float* corr, float* m,
                                               float* l) {
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g >= G) { corr[g] = 1.f; lg[g] = 0.f; continue; }
    float tm = lg[g];
    tm = fmaxf(tm, __shfl_xor(tm, 4));
    tm = fmaxf(tm, __shfl_xor(tm, 8));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m[g], tm);
    if (mn == -INFINITY) { corr[g] = 1.f; lg[g] = 0.f; continue; }
    corr[g] = exp2f(m[g] - mn);
    const float p = lg[g] == -INFINITY ? 0.f : exp2f(lg[g] - mn);
    const float ps = wave_sum((qq == 0) ? p : 0.f);
    l[g] = l[g] * corr[g] + ps;
    m[g] = mn;
    lg[g] = p;
  }
}

// Number of tokens of the token-by-token list of a sequence of length L: the
// bf16 sink [0, min(L, n_sink)), the INT2 head tail [n_sink, min(16 cf,
// int2_end)), the INT2 end tail [16 cl, int2_end) and the bf16 recent window
// [max(n_sink, L - W), L), in that order.
__device__ __forceinline__ int token_list_size(const DecodeArgs& a, int L, const Int2Range& rg) {
  const int n_sk = min(L, a.n_sink);
  const int n_hd = max(0, min(rg.cf * kChunkTokens, rg.int2_end) - a.n_sink);
  const int n_en = max(0, rg.int2_end - rg.cl * kChunkTokens);
  const int n_rc = max(0, L - max(a.n_sink, L - a.n_recent));
  return n_sk + n_hd + n_en + n_rc;
}

// Token-by-token path over 16-token tiles tile_first, tile_first + tile_step,
// ... (below tile_end) of that list, one tile per wave step, plain fp32.
// Lane (t, qq) dots 32 channels of token t's key with q' (LDS); the lane
// owns channels 2*lane, 2*lane+1 of o'.  INT2 tokens are dequantized in
// registers: key dot = s_K (q'.c) + z_K sum(q'), value = z_V + s_V c.
template <int GP>
__device__ void token_path(const DecodeArgs& a, int b, int h, int L, const Int2Range& rg,
                           int tile_first, int tile_end, int tile_step,
                           const float (*qs)[kHeadDim], const float* qsum,
                           float (*pbuf)[16][GP], float* m, float* l, float* acc0, float* acc1) {
  const int G = a.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = lane >> 2, qq = lane & 3;
  const int n_sk = min(L, a.n_sink);
  const int h_end = min(rg.cf * kChunkTokens, rg.int2_end);
  const int n_hd = max(0, h_end - a.n_sink);
  const int e_begin = rg.cl * kChunkTokens;
  const int n_en = max(0, rg.int2_end - e_begin);
  const int r_begin = max(a.n_sink, L - a.n_recent);
  const int n_rc = max(0, L - r_begin);
  const int n_all = n_sk + n_hd + n_en + n_rc;
  const int64_t sh_base = int64_t(b) * a.n_kv_heads + h;
  // position of virtual token idx
  auto position = [&](int idx) -> int {
    if (idx < n_sk) return idx;
    idx -= n_sk;
    if (idx < n_hd) return a.n_sink + idx;
    idx -= n_hd;
    if (idx < n_en) return e_begin + idx;
    return r_begin + (idx - n_en);
  };
  auto bf16_ptr = [&](int pos) -> const uint16_t* {
    if (pos < a.n_sink) return a.sink + (sh_base * a.n_sink + pos) * 2 * kHeadDim;
    return a.recent + (sh_base * a.n_recent + (pos - a.n_sink) % a.n_recent) * 2 * kHeadDim;
  };
  auto is_int2 = [&](int pos) { return pos >= a.n_sink && pos < rg.int2_end; };
  for (int tile = tile_first; tile < tile_end && tile * 16 < n_all; tile += tile_step) {
    const int idx = tile * 16 + t;
    const bool valid = idx < n_all;
    const int pos = position(valid ? idx : 0);
    // partial dot over this lane's 32 channels; the quad reduction follows
    float dot[GP], ksc = 1.f, kzr = 0.f;
#pragma unroll
    for (int g = 0; g < GP; ++g) dot[g] = 0.f;
    if (valid && is_int2(pos)) {
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, pos);
      const uint8_t* ch = a.pool + (off < 0 ? 0 : off);
      const int ts = pos % kChunkTokens;
      const uint2 kc = *reinterpret_cast<const uint2*>(ch + kKCodesOff + 32 * ts + 8 * qq);
      const uint32_t kp = *reinterpret_cast<const uint32_t*>(ch + kKParamsOff + 4 * ts);
      ksc = f16_bits_to_float(kp & 0xFFFFu);
      kzr = f16_bits_to_float(kp >> 16);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < G) {
          const float* qv = &qs[g][32 * qq];
#pragma unroll
          for (int k = 0; k < 16; ++k) dot[g] = fmaf(qv[k], float((kc.x >> (2 * k)) & 3u), dot[g]);
#pragma unroll
          for (int k = 0; k < 16; ++k) dot[g] = fmaf(qv[16 + k], float((kc.y >> (2 * k)) & 3u), dot[g]);
        }
      }
    } else if (valid) {
      const uint16_t* kp = bf16_ptr(pos) + 32 * qq;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < G) {
#pragma unroll
          for (int k = 0; k < 32; ++k) dot[g] = fmaf(qs[g][32 * qq + k], bf16_bits_to_float(kp[k]), dot[g]);
        }
      }
    }
    float lg[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float d = dot[g];
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      lg[g] = (valid && g < G) ? fmaf(ksc, d, kzr * qsum[g]) : -INFINITY;
    }
    float corr[GP];
    softmax_tile16<GP>(G, qq, lg, corr, m, l);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (qq == 0) pbuf[wave][t][g] = lg[g];
      acc0[g] *= corr[g];
      acc1[g] *= corr[g];
    }
    __builtin_amdgcn_wave_barrier();
    const int nt = min(16, n_all - tile * 16);
    float v0[16], v1[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {   // all loads first: one memory latency per tile
      v0[tt] = 0.f;
      v1[tt] = 0.f;
      if (tt < nt) {
        const int pp = position(tile * 16 + tt);
        if (is_int2(pp)) {
          const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                           a.page_size, b, h, pp);
          const uint8_t* ch = a.pool + (off < 0 ? 0 : off);
          const int ts = pp % kChunkTokens, cg = lane >> 1;
          const uint32_t byte = ch[kVCodesOff + 32 * (cg & 15) + 8 * (ts >> 2) + 4 * (cg >> 4) + (ts & 3)];
          const uint32_t vp = *reinterpret_cast<const uint32_t*>(ch + kVParamsOff + 4 * ts);
          const float sv = f16_bits_to_float(vp & 0xFFFFu), zv = f16_bits_to_float(vp >> 16);
          const int sh = 4 * (lane & 1);
          v0[tt] = fmaf(sv, float((byte >> sh) & 3u), zv);
          v1[tt] = fmaf(sv, float((byte >> (sh + 2)) & 3u), zv);
        } else {
          const uint32_t v2 = *reinterpret_cast<const uint32_t*>(bf16_ptr(pp) + kHeadDim + 2 * lane);
          v0[tt] = bf16_bits_to_float(v2 & 0xFFFFu);
          v1[tt] = bf16_bits_to_float(v2 >> 16);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float p = tt < nt ? pbuf[wave][tt][g] : 0.f;
        acc0[g] = fmaf(p, v0[tt], acc0[g]);
        acc1[g] = fmaf(p, v1[tt], acc1[g]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Merge the softmax states of the 4 waves of a work-group (m, l per head and
// unnormalized o'[128] per head, staged in LDS) and store the work-group's
// partial in slot `part_slot` of the workspace.  Then take an arrival ticket
// of (b, h); the last of its n_parts work-groups combines the partials in
// slots [base_slot, base_slot + n_parts), applies o = R_V o' and writes `out`.
template <int GP>
__device__ void finish_work_group(const DecodeArgs& a, int b, int h, int64_t part_slot,
                                  int64_t base_slot, int n_parts,
                                  float (*wm)[GP], float (*wl)[GP], float (*wo)[GP][kHeadDim],
                                  float (*ocomb)[kHeadDim], float (*s_m)[GP], float (*s_l)[GP]) {
  const int G = a.group;
  const int tid = threadIdx.x;
  const int64_t head = int64_t(b) * a.n_kv_heads + h;
  float* part = a.partials + part_slot * G * kPartialStride;
  // Merged partial -> LDS (wo[0] is free once every thread has read its
  // inputs), then one wave stores it, makes it visible device-wide (one
  // agent-scope release per work-group) and takes the arrival ticket.
  float* stage = &wo[0][0][0];
  float merged[(GP * kHeadDim + 255) / 256];
  float Ms[(GP * kHeadDim + 255) / 256], Ls[(GP * kHeadDim + 255) / 256];
#pragma unroll
  for (int k = 0; k < (GP * kHeadDim + 255) / 256; ++k) {
    const int i = tid + 256 * k;
    merged[k] = 0.f;
    Ms[k] = -INFINITY;
    Ls[k] = 0.f;
    if (i < G * kHeadDim) {
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
      merged[k] = o;
      Ms[k] = M;
      Ls[k] = l;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (GP * kHeadDim + 255) / 256; ++k) {
    const int i = tid + 256 * k;
    if (i < G * kHeadDim) {
      const int g = i / kHeadDim, c = i % kHeadDim;
      stage[g * kPartialStride + 4 + c] = merged[k];
      if (c == 0) {
        stage[g * kPartialStride + 0] = Ms[k];
        stage[g * kPartialStride + 1] = Ls[k];
      }
    }
  }
  __syncthreads();
  __shared__ int is_last;
  if (tid < 64) {
    for (int i = tid; i < G * kPartialStride; i += 64) store_agent(part + i, stage[i]);
    wait_global_stores();   // the partial is complete before the ticket is taken
    if (tid == 0) {
      const int prev = fetch_add_agent(&a.tickets[head], 1);
      is_last = (prev == n_parts - 1);
    }
  }
  __syncthreads();
  if (!is_last) return;
  // Every other partial of (b, h) is complete; they are read with
  // device-coherent loads below.

  // Split weights f_i = 2^(m_i - M) / sum_k 2^(m_k - M) l_k, staged in LDS
  // in slices of kCombineSlice splits so that all loads of a slice are in
  // flight together.
  const float* base = a.partials + base_slot * G * kPartialStride;
  // s_m, s_l: [kCombineSlice][GP] staging of the split weights (caller's LDS)
  __shared__ float s_M[GP], s_den[GP];
  const int wave = tid >> 6, lane = tid & 63;
  if (tid < GP) { s_M[tid] = -INFINITY; s_den[tid] = 0.f; }
  __syncthreads();
  for (int s0 = 0; s0 < n_parts; s0 += kCombineSlice) {      // pass 1: M per head
    const int ns = min(kCombineSlice, n_parts - s0);
    for (int i = tid; i < ns * G; i += blockDim.x) {
      const float* p = base + ((s0 + i / G) * G + i % G) * kPartialStride;
      s_m[i / G][i % G] = load_agent(p);
    }
    __syncthreads();
    for (int g = wave; g < G; g += 4) {
      float mx = -INFINITY;
      for (int i = lane; i < ns; i += 64) mx = fmaxf(mx, s_m[i][g]);
      mx = wave_max(mx);
      if (lane == 0) s_M[g] = fmaxf(s_M[g], mx);
    }
    __syncthreads();
  }
  constexpr int KO = (GP * kHeadDim + 255) / 256;             // outputs per thread
  float acc[KO];
#pragma unroll
  for (int k = 0; k < KO; ++k) acc[k] = 0.f;
  for (int s0 = 0; s0 < n_parts; s0 += kCombineSlice) {      // pass 2: weighted sums
    const int ns = min(kCombineSlice, n_parts - s0);
    for (int i = tid; i < ns * G; i += blockDim.x) {
      const float* p = base + ((s0 + i / G) * G + i % G) * kPartialStride;
      const float M = s_M[i % G];
      const float f = M == -INFINITY ? 0.f : exp2f(load_agent(p) - M);
      s_m[i / G][i % G] = f;
      s_l[i / G][i % G] = f * load_agent(p + 1);
    }
    __syncthreads();
    for (int g = wave; g < G; g += 4) {
      float dn = 0.f;
      for (int i = lane; i < ns; i += 64) dn += s_l[i][g];
      dn = wave_sum(dn);
      if (lane == 0) s_den[g] += dn;
    }
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int o = tid + k * blockDim.x;
      if (o < G * kHeadDim) {
        const int g = o / kHeadDim, c = o % kHeadDim;
        float v = 0.f;
#pragma unroll 8
        for (int i = 0; i < ns; ++i)
          v = fmaf(s_m[i][g], load_agent(base + ((s0 + i) * G + g) * kPartialStride + 4 + c), v);
        acc[k] += v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int o = tid + k * blockDim.x;
    if (o < G * kHeadDim) {
      const int g = o / kHeadDim, c = o % kHeadDim;
      ocomb[g][c] = s_den[g] > 0.f ? acc[k] / s_den[g] : 0.f;
    }
  }
  __syncthreads();
  // o = R_V o' (row-major R_V: o_i = sum_j R_V[i][j] o'_j)
  const float* R = a.R_V + int64_t(h) * kHeadDim * kHeadDim;
  for (int i = tid; i < G * kHeadDim; i += blockDim.x) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    const float4* row = reinterpret_cast<const float4*>(R + c * kHeadDim);
    float o = 0.0f;
#pragma unroll 4
    for (int j = 0; j < kHeadDim / 4; ++j) {
      const float4 r = row[j];
      o = fmaf(r.x, ocomb[g][4 * j + 0], o);
      o = fmaf(r.y, ocomb[g][4 * j + 1], o);
      o = fmaf(r.z, ocomb[g][4 * j + 2], o);
      o = fmaf(r.w, ocomb[g][4 * j + 3], o);
    }
    a.out[(int64_t(b) * a.n_q_heads + h * G + g) * kHeadDim + c] = o;
  }
  if (tid == 0) store_agent(&a.tickets[head], 0);   // ready for the next call on this workspace
}

}  // namespace kvq
