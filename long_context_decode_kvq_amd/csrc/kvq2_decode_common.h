// Pieces shared by the decode kernels: the kernel arguments, the INT2
// range and token-list geometry, the token-by-token tile, the work-group
// merge of per-wave softmax states, the split-K partial store and the
// combines with the output inverse rotation (per (b, h) or per query head
// for the MFMA decode, last-arrival for the VALU decode).
//
// OSCAR technical summary, sec. 2.2-B: the fused kernel undoes the rotation;
// here that is done exactly once per query head on each side: q' = R_K^T q
// before the token loop and o = R_V o' after the split-K combine.
#pragma once

#include "kvq2_device.h"

namespace kvq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCombineSlice = 64;   // splits staged per combine pass

// Words of one state of the self-calibrating range weights: the sums of
// range durations (s_memrealtime ticks) per (dispatch round r, XCD x) at
// kFbSum + 8 r + x, their counts at kFbCnt + 8 r + x, then the current XCD
// and round weights (1/1024 units; 0 before the first update).  One state
// per (G <= 4 or G = 8, 2 .. 4 rounds).
constexpr int kFbSum = 0, kFbCnt = 32, kFbXw = 64, kFbRw = 72, kFbWords = 80;
constexpr int kFbStates = 6;

struct DecodeArgs {
  const float* R_K;
  const float* R_V;
  const uint8_t* pool;
  int64_t num_pages;
  const uint16_t* sink;
  const uint16_t* recent;
  const int32_t* block_table;
  int32_t bt_stride;
  int n_q_heads, n_kv_heads, page_size, n_sink, n_recent;
  // Rows of one (sequence, KV head): the head_group = Hq / Hkv query heads
  // of each of the n_query queries this launch takes, queries query_base ..
  // query_base + n_query - 1 of the query_count queries of every sequence
  // (1 for decode; M for multi-query attention, whose queries sit at the
  // sequence's last M positions).  Row r is query query_base + r /
  // head_group, head h head_group + r % head_group; group = n_query *
  // head_group rows share the KV head's tiles (the MFMA decode's "heads" are
  // these rows).
  int group, head_group, n_query, query_base, query_count;
  float alpha;                 // sm_scale * log2(e): logits are kept in base-2 units
  float sigma_v;               // power of two with sigma_v * s_V <= 1 for every V scale
  int log2_sigma_v;            // log2(sigma_v)
  int log2_cpp;                // log2(page_size / 16)
  int ng;                      // (scale, zero) pairs per vector: quantization groups of 128 / ng
  int chunk_bytes;             // bytes of one 16-token chunk: 1024 + 128 ng
  int64_t page_bytes;          // bytes of one physical page: Hkv * page_size / 16 * chunk_bytes
  const int32_t* seq_len;
  const uint16_t* q;
  float* out;
  int32_t* tickets;            // [B * Hkv] (VALU decode)
  int batch;
  float* qrot;                 // [B][Hq][kQStride]: alpha R_K^T q, its sum, f16 exponent
  uint32_t* bq;                // [B * Hkv][kBqWords]: QK MFMA operand and lane constants
  int gp;                      // MFMA head-group width (2, 4 or 8)
  float* partials;             // MFMA: slots [range + pair], then token-list slices;
                               // VALU: [B][Hkv][n_split]; each slot [G][kPartialStride]
  int n_split_int2;            // VALU decode: even INT2 splits per (b, h)
  int n_split;                 // VALU decode: n_split_int2 + the bf16 work-group
  // MFMA decode: tile_prefix[b] = sum over b' < b of W_b' (B + 1 entries,
  // written by the pre-pass), W_b = max(1, INT2 tiles of sequence b) +
  // piece_cost; the launch cuts the concatenated W_b of all (b, h) into equal
  // ranges, one per work-group.  piece_cost virtual tiles at the start of
  // every (b, h) stand for the fixed cost of one more piece (prologue,
  // partial, combine), so that a work-group that starts a pair streams fewer
  // tiles.
  int32_t* tile_prefix;
  int piece_cost;
  // MFMA decode: the cut into chain_groups ranges, written by the pre-pass:
  // range i is virtual tiles [range_start[i], range_start[i + 1]) (chain_groups
  // + 1 entries), and pair_range[b Hkv + h] = i0 | i1 << 16, the first and
  // last range that touch (b, h).  Ranges are sized by round_weight (1/1024
  // units) of the work-group's dispatch round i / round_size: the work-groups
  // of one CU stream at different rates by dispatch order.
  int32_t* range_start;
  int32_t* pair_range;
  // Self-calibrating range weights (kFb* layout below), or null: each range
  // work-group adds its duration to the cell (round, XCD) of its index, and
  // the next call's plan moves the weights toward equal durations.
  uint32_t* feedback;
  int chain_groups;
  int round_size;
  int round_weight[4];
  // Weight of a work-group's range by the XCD it runs on (work-group i is
  // dispatched to XCD i mod 8), 1/1024 units.
  int xcd_weight[8];
  // MFMA decode: the token-by-token list of (b, h) is cut into n_tok_slices
  // slices of 64 tokens; the pre-pass leaves the partial of slice z in slot
  // tok_slot0 + (b Hkv + h) n_tok_slices + z, and the combine takes them in.
  int n_tok_slices;
  int64_t tok_slot0;
  // MFMA decode with shared-prefix groups (n_groups > 0): the caller's
  // groups, and the pre-pass's resolution of them.  A valid member b of
  // group j skips its first seq_skip[b] INT2 tiles, which the group's
  // row-set items read for up to four members at once; their partials are
  // in slots rs_slot0 + 4 (range + item) + member % 4.
  int n_groups;
  int n_members;
  int rs_cost;                 // virtual tiles per row-set tile
  const int32_t* member_start; // [n_groups + 1]
  const int32_t* members;      // [n_members]
  const int32_t* prefix_len;   // [n_groups]
  int32_t* seq_skip;           // [B] tiles read by the member's group (0: none)
  int32_t* seq_member;         // [B] first member index listing b
  int32_t* seq_group;          // [B] group of a valid member, else -1
  int32_t* grp_info;           // [n_groups][kGrpInfo]
  int32_t* item_range;         // per row-set item: first | last range << 16
  int64_t rs_slot0;
};

// Row of grp_info per shared-prefix group (kGrpInfo ints, written by the
// pre-pass).
constexpr int kGiRsPrefix = 0;     // virtual tiles of the row-set items of earlier groups
constexpr int kGiWidth = 1;        // virtual tiles per item of this group
constexpr int kGiSkip = 2;         // prefix tiles (0 when no member is valid)
constexpr int kGiRep = 3;          // representative sequence (a valid member, else 0)
constexpr int kGiRowSets = 4;      // row sets (of four members) per KV head
constexpr int kGiItemBase = 5;     // index of the group's first item
constexpr int kGiMemberStart = 6;  // member range, clamped
constexpr int kGiMemberEnd = 7;

// INT2 work of a sequence of length L is split in two parts:
//  * whole tiles of `npt` fully valid 16-token chunks [cf, cl), streamed in
//    contiguous tile ranges;
//  * the few INT2 positions outside them (the partial chunk after the sink,
//    the partial chunk before the recent window and a sub-tile remainder),
//    which are handled token by token with the bf16 segments.
struct Int2Range {
  int int2_end;   // INT2 positions are [n_sink, int2_end)
  int cf, cl;     // tiled chunks [cf, cl), cl - cf a multiple of npt
};

// Element offset of row r of (b, h) in q and out, both [B][query_count][Hq][128].
__device__ __forceinline__ int64_t row_offset(const DecodeArgs& a, int b, int h, int r) {
  const int m = r / a.head_group, g = r - m * a.head_group;
  return ((int64_t(b) * a.query_count + a.query_base + m) * a.n_q_heads +
          int64_t(h) * a.head_group + g) * kHeadDim;
}

// First rotated-query record of (b, h) in qrot ([B][Hkv][rows][kQStride]).
__device__ __forceinline__ int64_t qrot_offset(const DecodeArgs& a, int b, int h) {
  return (int64_t(b) * a.n_kv_heads + h) * a.group * kQStride;
}

__device__ __forceinline__ Int2Range int2_range(const DecodeArgs& a, int L, int npt) {
  Int2Range r;
  r.int2_end = max(a.n_sink, L - a.n_recent);
  r.cf = (a.n_sink + kChunkTokens - 1) / kChunkTokens;
  const int full_end = r.int2_end / kChunkTokens;
  r.cl = full_end > r.cf ? r.cf + npt * ((full_end - r.cf) / npt) : r.cf;
  return r;
}

// Tile range [t_begin, t_end) of INT2 split s of n_split_int2 even splits.
__device__ __forceinline__ void split_tiles(const DecodeArgs& a, const Int2Range& r, int npt, int s,
                                            int& t_begin, int& t_end) {
  const int n = (r.cl - r.cf) / npt;
  t_begin = int(int64_t(n) * s / a.n_split_int2);
  t_end = int(int64_t(n) * (s + 1) / a.n_split_int2);
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
  const float* src = a.qrot + qrot_offset(a, b, h);
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
// leaves p = exp2(logit - m) in lg.  All 64 lanes must be active.
template <int GP>
__device__ __forceinline__ void softmax_tile16(int G, int qq, float* lg, float* corr, float* m,
                                               float* l) {
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g >= G) { corr[g] = 1.f; lg[g] = 0.f; continue; }
    // the lanes of a token hold equal values, so the two mirrors pair the
    // tokens of a row as xor 1 and xor 2 over t would
    float tm = lg[g];
    tm = fmaxf(tm, dpp_move<kRowHalfMirror>(tm));
    tm = fmaxf(tm, dpp_move<kRowMirror>(tm));
    tm = fmaxf(fmaxf(read_lane(tm, 0), read_lane(tm, 16)), fmaxf(read_lane(tm, 32), read_lane(tm, 48)));
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

// The token-by-token list of a sequence of length L, in this order: the
// bf16 sink [0, min(L, n_sink)), the INT2 head tail [n_sink, min(16 cf,
// int2_end)), the INT2 end tail [16 cl, int2_end) and the bf16 recent window
// [max(n_sink, L - W), L).
struct TokenList {
  int n_sk, n_hd, n_en, n_all, e_begin, r_begin, L;
};

__device__ __forceinline__ TokenList token_list(const DecodeArgs& a, int L, const Int2Range& rg) {
  TokenList t;
  t.n_sk = min(L, a.n_sink);
  t.n_hd = max(0, min(rg.cf * kChunkTokens, rg.int2_end) - a.n_sink);
  t.e_begin = rg.cl * kChunkTokens;
  t.n_en = max(0, rg.int2_end - t.e_begin);
  t.r_begin = max(a.n_sink, L - a.n_recent);
  t.n_all = t.n_sk + t.n_hd + t.n_en + max(0, L - t.r_begin);
  t.L = L;
  return t;
}

// Position of entry idx of the list.
__device__ __forceinline__ int token_position(const DecodeArgs& a, const TokenList& t, int idx) {
  if (idx < t.n_sk) return idx;
  idx -= t.n_sk;
  if (idx < t.n_hd) return a.n_sink + idx;
  idx -= t.n_hd;
  if (idx < t.n_en) return t.e_begin + idx;
  return t.r_begin + (idx - t.n_en);
}

// Global-memory byte pointer (a plain pointer rebuilt from integers would be
// generic, and its loads would count against the LDS wait counter too).
typedef const uint8_t __attribute__((address_space(1))) global_u8;

__device__ __forceinline__ global_u8* read_lane_ptr(const uint8_t* p, int lane) {
  const uint64_t u = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
  return reinterpret_cast<global_u8*>((uint64_t(hi) << 32) | lo);
}

// Entries [16 tile, 16 tile + 16) of the token-by-token list of (b, h),
// plain fp32 (one wave).  Lane (t, qq) = (lane / 4, lane % 4) dots channels
// 32 qq .. 32 qq + 31 of token t's key with q' (LDS); the lane owns
// channels 2 lane, 2 lane + 1 of o'.  Every key and value load of the tile is
// issued before the first use.  INT2 tokens are dequantized in registers:
// key dot = s_K (q'.c) + z_K sum(q'), value = z_V + s_V c.  pb: the wave's
// [16][GP] LDS buffer of softmax weights.  All 64 lanes must be active.
template <int GP>
__device__ void token_tile(const DecodeArgs& a, int b, int h, const TokenList& tl,
                           const Int2Range& rg, int tile, const float (*qs)[kHeadDim],
                           const float* qsum, const float (*qsum4)[4], float (*pb)[GP], float* m,
                           float* l, float* acc0, float* acc1) {
  const int nt = min(16, tl.n_all - tile * 16);
  if (nt <= 0) return;
  const int G = a.group;
  const int lane = threadIdx.x & 63, t = lane >> 2, qq = lane & 3;
  const int64_t sh = int64_t(b) * a.n_kv_heads + h;
  // token t: kind (0 none, 1 bf16 row, 2 INT2 chunk slot ts) and base address
  int kind = 0, ts = 0, pos = 0;
  const uint8_t* base = a.pool;
  if (t < nt) {
    pos = token_position(a, tl, tile * 16 + t);
    if (pos >= a.n_sink && pos < rg.int2_end) {
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, pos, a.chunk_bytes);
      kind = 2;
      ts = pos % kChunkTokens;
      base = a.pool + (off < 0 ? 0 : off);   // an invalid page entry reads chunk 0 (memory-safe)
    } else {
      kind = 1;
      const uint16_t* row =
          pos < a.n_sink ? a.sink + (sh * a.n_sink + pos) * 2 * kHeadDim
                         : a.recent + (sh * a.n_recent + (pos - a.n_sink) % a.n_recent) * 2 * kHeadDim;
      base = reinterpret_cast<const uint8_t*>(row);
    }
  }
  // ---- loads: the key part of token t, then the values of all 16 tokens.
  // Every load is issued on every path (tokens of the other kind, and
  // entries past the list, read harmless in-bounds bytes that are not used),
  // so that no branch separates a load from the next one.
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef const uint32_t __attribute__((address_space(1))) global_u32;
  typedef const u32x2 __attribute__((address_space(1))) global_u2;
  typedef const u32x4 __attribute__((address_space(1))) global_u4;
  global_u8* gbase = reinterpret_cast<global_u8*>(reinterpret_cast<uintptr_t>(base));
  global_u8* gpool = reinterpret_cast<global_u8*>(reinterpret_cast<uintptr_t>(a.pool));
  u32x4 kb[4];
  {
    global_u4* p = reinterpret_cast<global_u4*>(kind == 1 ? gbase + 64 * qq : gpool);
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = p[i];
  }
  u32x2 kc = *reinterpret_cast<global_u2*>(kind == 2 ? gbase + kKCodesOff + 32 * ts + 8 * qq
                                                           : gpool);
  // (s_K, z_K) of the quantization group of this lane's 32 key channels
  const int ng = a.ng;
  uint32_t kpar = *reinterpret_cast<global_u32*>(
      kind == 2 ? gbase + param_offset(0, ts, ng, (qq * ng) >> 2) : gpool);
  // Values: one dword per lane and token (bf16: channels 2 lane, 2 lane + 1
  // of the value row; INT2: the dword holding this lane's code byte), and
  // for INT2 tokens the (s_V, z_V) pair of the lane's value group.  Every
  // one is a vector load on one path: a scalar load under a branch on the
  // group count made the compiler wait for all earlier vector loads before
  // each token's, sixteen memory latencies per tile.
  uint32_t vword[16], vpar[16];
  int vkind[16];
  const int cg = lane >> 1, vgrp = (lane * ng) >> 6;
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    vkind[tt] = __builtin_amdgcn_readlane(kind, 4 * tt);
    const int s = __builtin_amdgcn_readlane(ts, 4 * tt);
    global_u8* bp = read_lane_ptr(base, 4 * tt);
    const int boff = kVCodesOff + 32 * (cg & 15) + 8 * (s >> 2) + 4 * (cg >> 4);   // + (s & 3)
    const int woff = vkind[tt] == 1 ? 2 * kHeadDim + 4 * lane : boff;
    vword[tt] = *reinterpret_cast<global_u32*>(bp + woff);
    vpar[tt] = *reinterpret_cast<global_u32*>(vkind[tt] == 2 ? bp + param_offset(1, s, ng, vgrp)
                                                               : gpool);
  }
  // Empty asm statements take the loaded values here: the compiler would
  // otherwise sink each load into the branch that uses it, one wait per load.
  asm volatile("" : "+v"(kb[0]), "+v"(kb[1]), "+v"(kb[2]), "+v"(kb[3]), "+v"(kc), "+v"(kpar));
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) asm volatile("" : "+v"(vword[tt]), "+v"(vpar[tt]));
  // ---- logits
  float dot[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) dot[g] = 0.f;
  if (kind == 1) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g < G) {
        const float* qv = &qs[g][32 * qq];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w[4] = {kb[i].x, kb[i].y, kb[i].z, kb[i].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            dot[g] = fmaf(qv[8 * i + 2 * k], bf16_bits_to_float(w[k] & 0xFFFFu), dot[g]);
            dot[g] = fmaf(qv[8 * i + 2 * k + 1], bf16_bits_to_float(w[k] >> 16), dot[g]);
          }
        }
      }
    }
  } else if (kind == 2) {
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
  }
  const float ksc = kind == 2 ? f16_bits_to_float(kpar & 0xFFFFu) : 1.f;
  const float kzr = kind == 2 ? f16_bits_to_float(kpar >> 16) : 0.f;
  float lg[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float d = dot[g];
    // with several key groups each lane scales its own 32 channels (the
    // logit is the quad sum of s_K (q'.c) + z_K sum(q') over the groups)
    if (ng > 1 && kind == 2 && g < G) d = fmaf(ksc, d, kzr * qsum4[g][qq]);
    d += dpp_move<kQuadXor1>(d);
    d += dpp_move<kQuadXor2>(d);
    // row g's query sits at position L - query_count + query_base + g /
    // head_group and sees the positions up to it (with query_count <=
    // n_recent only recent-window tokens can lie beyond it; for decode every
    // position is visible)
    const bool seen = pos <= tl.L - a.query_count + a.query_base + g / a.head_group;
    const float logit = (kind == 2 && ng == 1) ? fmaf(ksc, d, kzr * qsum[g]) : d;
    lg[g] = (kind != 0 && g < G && seen) ? logit : -INFINITY;
  }
  float corr[GP];
  softmax_tile16<GP>(G, qq, lg, corr, m, l);
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (qq == 0) pb[t][g] = lg[g];
    acc0[g] *= corr[g];
    acc1[g] *= corr[g];
  }
  __builtin_amdgcn_wave_barrier();
  // ---- values: o' += p v over the tile's tokens
  const int vsh = 4 * (lane & 1);
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    if (vkind[tt] == 0) continue;
    float v0, v1;
    if (vkind[tt] == 1) {
      v0 = bf16_bits_to_float(vword[tt] & 0xFFFFu);
      v1 = bf16_bits_to_float(vword[tt] >> 16);
    } else {
      const float sv = f16_bits_to_float(vpar[tt] & 0xFFFFu), zv = f16_bits_to_float(vpar[tt] >> 16);
      const uint32_t byte = vword[tt] >> (8 * (__builtin_amdgcn_readlane(ts, 4 * tt) & 3));
      v0 = fmaf(sv, float((byte >> vsh) & 3u), zv);
      v1 = fmaf(sv, float((byte >> (vsh + 2)) & 3u), zv);
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float p = pb[tt][g];
      acc0[g] = fmaf(p, v0, acc0[g]);
      acc1[g] = fmaf(p, v1, acc1[g]);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Merge the softmax states (m, l per head, unnormalized o'[128] per head) of
// the 4 waves of a work-group, staged in LDS, into stage[g * kPartialStride
// + ...] = (M, l, 2 pad, o'[128]) (stage may alias wo[0]).  Ends with a
// barrier.
template <int GP>
__device__ void merge_wave_states(int G, const float (*wm)[GP], const float (*wl)[GP],
                                  float (*wo)[GP][kHeadDim], float* stage) {
  const int tid = threadIdx.x;
  constexpr int K = (GP * kHeadDim + 255) / 256;
  float merged[K], Ms[K], Ls[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
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
  for (int k = 0; k < K; ++k) {
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
}

// Merge the 4 waves' states (as merge_wave_states) straight into the
// work-group's partial `part` in the workspace: (M, l, 2 pad, o'[128]) per
// head, plain stores (read by a later kernel).  The LDS inputs stay intact.
template <int GP>
__device__ void store_partial(int G, const float (*wm)[GP], const float (*wl)[GP],
                              const float (*wo)[GP][kHeadDim], float* part) {
  const int tid = threadIdx.x;
  constexpr int K = (GP * kHeadDim + 255) / 256;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int i = tid + 256 * k;
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
      part[g * kPartialStride + 4 + c] = o;
      if (c == 0) {
        part[g * kPartialStride + 0] = M;
        part[g * kPartialStride + 1] = l;
      }
    }
  }
}
// The four waves' partials of a row-set piece, each for its own member's
// query rows: wave w's G rows go to the slot after wave w - 1's.
template <int GP>
__device__ void store_wave_partials(int G, const float (*wm)[GP], const float (*wl)[GP],
                                    const float (*wo)[GP][kHeadDim], float* part) {
  for (int i = threadIdx.x; i < 4 * G * kHeadDim; i += blockDim.x) {
    const int w = i / (G * kHeadDim), r = i % (G * kHeadDim);
    const int g = r / kHeadDim, c = r % kHeadDim;
    float* pw = part + (w * G + g) * kPartialStride;
    pw[4 + c] = wo[w][g][c];
    if (c == 0) {
      pw[0] = wm[w][g];
      pw[1] = wl[w][g];
    }
  }
}

// The row-set partials of (b, h) in a shared-prefix decode: returns their
// count and sets `first` to the first one's slot (the others follow four
// slots apart); 0 when b reads its whole cache itself.
__device__ __forceinline__ int rowset_slots(const DecodeArgs& a, int b, int h, int64_t& first) {
  first = 0;
  if (a.n_groups <= 0) return 0;
  const int gidx = a.seq_group[b];
  if (gidx < 0) return 0;
  const int32_t* gi = a.grp_info + int64_t(gidx) * kGrpInfo;
  const int m = a.seq_member[b] - gi[kGiMemberStart];
  const int64_t q = gi[kGiItemBase] + int64_t(h) * gi[kGiRowSets] + m / 4;
  const int ir = a.item_range[q];
  const int i0 = ir & 0xFFFF, i1 = ir >> 16;
  first = a.rs_slot0 + (int64_t(i0) + q) * 4 + m % 4;
  return i1 - i0 + 1;
}

// Split-K combine of one (b, h), by a work-group of NT (256 or 512) threads in a kernel
// of its own: the partials in slots [base_slot, base_slot + n_parts) and
// [tok_slot, tok_slot + n_tok), with M = max m_s, f_s = 2^(m_s - M):
// o' = sum f_s o'_s / sum f_s l_s, then o = R_V o' to `out`.  The slots are
// taken in slices of kSlice (the running M, l and o' are rescaled between
// slices).  Every load of a slice is issued before any is used, and R_V
// after the first slice's: the wait for a slice then leaves R_V in flight,
// so the call's critical path is one round trip to the partials.  The (m, l)
// of a slice are staged in LDS per head, read back as vectors.
template <int GP, bool RSL = false, int NT = 256>
__device__ void combine_pair(const DecodeArgs& a, int b, int h, int64_t base_slot, int n_parts,
                             int64_t tok_slot, int n_tok, int64_t rs_slot = 0, int n_rs = 0) {
  constexpr int kSlice = 16;
  constexpr int KO = (GP * kHeadDim + NT - 1) / NT;   // outputs per thread
  constexpr int NS = NT / kHeadDim;                   // parts of an R_V row
  constexpr int RC = kHeadDim / NS;                   // R_V columns per thread
  __shared__ __attribute__((aligned(16))) float s_m[GP][kSlice];
  __shared__ __attribute__((aligned(16))) float s_l[GP][kSlice];
  __shared__ __attribute__((aligned(16))) float ocomb[GP][kHeadDim];
  __shared__ float red[NS][GP][kHeadDim];
  const int G = a.group;
  const int tid = threadIdx.x;
  const int ri = tid & (kHeadDim - 1), part = tid / kHeadDim;
  auto slot_ptr = [&](int i) -> const float* {
    int64_t s = i < n_parts ? base_slot + i : tok_slot + (i - n_parts);
    if constexpr (RSL) s = i < n_parts + n_tok ? s : rs_slot + 4 * int64_t(i - n_parts - n_tok);
    return a.partials + s * G * kPartialStride;
  };
  int gk[KO], ck[KO];
  float M[KO], den[KO], acc[KO];
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int o = tid + NT * k;
    gk[k] = min(o / kHeadDim, G - 1);   // rows past G load head G - 1 and are not stored
    ck[k] = o % kHeadDim;
    M[k] = -INFINITY;
    den[k] = 0.f;
    acc[k] = 0.f;
  }
  const int n_all = n_parts + n_tok + (RSL ? n_rs : 0);
  float ov[kSlice][KO];
  float2 ml = {-INFINITY, 0.f};
  // issue the loads of slice s0 (ns > 0 slots): thread (i, g), i < ns, takes
  // the (m, l) of slot i, head g
  auto load_slice = [&](int s0, int ns) {
#pragma unroll
    for (int i = 0; i < kSlice; ++i) {
      const float* p = slot_ptr(s0 + min(i, ns - 1));   // past the slice: re-read, unused
#pragma unroll
      for (int k = 0; k < KO; ++k) ov[i][k] = p[gk[k] * kPartialStride + 4 + ck[k]];
    }
    if (tid < ns * G)
      ml = *reinterpret_cast<const float2*>(slot_ptr(s0 + tid / G) + (tid % G) * kPartialStride);
  };
  if (n_all > 0) load_slice(0, min(kSlice, n_all));
  // keep R_V's loads behind the slice's in issue order
  asm volatile("" ::: "memory");
  float4 r[RC / 4];
  {
    const float4* row = reinterpret_cast<const float4*>(
        a.R_V + int64_t(h) * kHeadDim * kHeadDim + ri * kHeadDim + RC * part);
#pragma unroll
    for (int j = 0; j < RC / 4; ++j) r[j] = row[j];
  }
  for (int s0 = 0; s0 < n_all; s0 += kSlice) {
    const int ns = min(kSlice, n_all - s0);
    if (s0 > 0) load_slice(s0, ns);
    if (tid < ns * G) {
      s_m[tid % G][tid / G] = ml.x;
      s_l[tid % G][tid / G] = ml.y;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int g = gk[k];
      float mv[kSlice], lv[kSlice];
#pragma unroll
      for (int i = 0; i < kSlice; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&s_m[g][i]);
        const float4 y = *reinterpret_cast<const float4*>(&s_l[g][i]);
        mv[i] = x.x; mv[i + 1] = x.y; mv[i + 2] = x.z; mv[i + 3] = x.w;
        lv[i] = y.x; lv[i + 1] = y.y; lv[i + 2] = y.z; lv[i + 3] = y.w;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kSlice; ++i) mx = i < ns ? fmaxf(mx, mv[i]) : mx;
      const float nM = fmaxf(M[k], mx);
      if (nM != -INFINITY) {
        const float sc = M[k] == -INFINITY ? 0.f : exp2f(M[k] - nM);
        acc[k] *= sc;
        den[k] *= sc;
#pragma unroll
        for (int i = 0; i < kSlice; ++i) {
          const float f = (i >= ns || mv[i] == -INFINITY) ? 0.f : exp2f(mv[i] - nM);
          acc[k] = fmaf(f, ov[i][k], acc[k]);
          den[k] = fmaf(f, lv[i], den[k]);
        }
        M[k] = nM;
      }
    }
    __syncthreads();   // s_m, s_l are refilled by the next slice
  }
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int o = tid + NT * k;
    if (o < G * kHeadDim) ocomb[gk[k]][ck[k]] = den[k] > 0.f ? acc[k] / den[k] : 0.f;
  }
  __syncthreads();
  // o = R_V o' (row-major R_V: o_i = sum_j R_V[i][j] o'_j); thread (part, i)
  // holds one of NS parts of row i and applies it to every head; the parts
  // meet in LDS.
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < G) {
      const float* oc = &ocomb[g][RC * part];
      float o = 0.f;
#pragma unroll
      for (int j = 0; j < RC / 4; ++j) {
        o = fmaf(r[j].x, oc[4 * j + 0], o);
        o = fmaf(r[j].y, oc[4 * j + 1], o);
        o = fmaf(r[j].z, oc[4 * j + 2], o);
        o = fmaf(r[j].w, oc[4 * j + 3], o);
      }
      red[part][g][ri] = o;
    }
  }
  __syncthreads();
  for (int k = tid; k < G * kHeadDim; k += NT) {
    const int g = k / kHeadDim, c = k % kHeadDim;
    float o = red[0][g][c];
#pragma unroll
    for (int q = 1; q < NS; ++q) o += red[q][g][c];
    a.out[row_offset(a, b, h, g) + c] = o;
  }
}

// Split-K combine of one query head g of (b, h), by a work-group of NQ x 128
// threads in a kernel of its own (one work-group per query head, so that a
// small batch still spreads its combines over many CUs): the partials in
// slots [base_slot, base_slot + n_parts) and [tok_slot, tok_slot + n_tok),
// with M = max m_s, f_s = 2^(m_s - M): o' = sum f_s o'_s / sum f_s l_s, then
// o = R_V o' to `out`.  Thread (part, c) takes channel c of the slots of its
// part of each round (kRound slots per part, all loads in flight together;
// the (m, l) of a round are staged in LDS once), and the NQ parts merge in
// LDS; R_V row c, 128 / NQ columns per thread, is loaded right after the
// first round, so that the wait for the round leaves it in flight.  With NQ = 8
// a round covers 128 slots: the split count of a batch-1 decode (about 70)
// takes one round of dependent loads instead of three.
template <int GP, int NQ, bool RSL = false>
__device__ void combine_head(const DecodeArgs& a, int b, int h, int g, int64_t base_slot,
                             int n_parts, int64_t tok_slot, int n_tok, int64_t rs_slot = 0,
                             int n_rs = 0) {
  constexpr int kRound = 16;              // slots per part per round
  constexpr int kCols = kHeadDim / NQ;    // R_V columns per thread
  __shared__ float s_ml[NQ * kRound][2];
  __shared__ float s_part[NQ][3][kHeadDim];   // per part: M, den, acc
  __shared__ float ocomb[kHeadDim];
  __shared__ float red[NQ][kHeadDim];
  const int G = a.group;
  const int tid = threadIdx.x;
  const int c = tid & (kHeadDim - 1), part = tid >> 7;
  auto slot_ptr = [&](int i) -> const float* {
    int64_t s = i < n_parts ? base_slot + i : tok_slot + (i - n_parts);
    if constexpr (RSL) s = i < n_parts + n_tok ? s : rs_slot + 4 * int64_t(i - n_parts - n_tok);
    return a.partials + (s * G + g) * kPartialStride;
  };
  const int n_all = n_parts + n_tok + (RSL ? n_rs : 0);
  float ov[kRound];
  float mlv = 0.f;
  // issue the loads of round s0 (ns > 0 slots)
  auto load_round = [&](int s0, int ns) {
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      const int i = part * kRound + k;
      ov[k] = slot_ptr(s0 + min(i, ns - 1))[4 + c];   // past the round: re-read, unused
    }
    if (tid < 2 * ns) mlv = slot_ptr(s0 + (tid >> 1))[tid & 1];
  };
  if (n_all > 0) load_round(0, min(NQ * kRound, n_all));
  // keep R_V's loads behind the first round's in issue order
  asm volatile("" ::: "memory");
  float4 r[kCols / 4];
  {
    const float4* row = reinterpret_cast<const float4*>(
        a.R_V + int64_t(h) * kHeadDim * kHeadDim + c * kHeadDim + kCols * part);
#pragma unroll
    for (int j = 0; j < kCols / 4; ++j) r[j] = row[j];
  }
  float M = -INFINITY, den = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_all; s0 += NQ * kRound) {
    const int ns = min(NQ * kRound, n_all - s0);
    if (s0 > 0) load_round(s0, ns);
    if (tid < 2 * ns) s_ml[tid >> 1][tid & 1] = mlv;
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
      const int i = part * kRound + k;
      if (i < ns) mx = fmaxf(mx, s_ml[i][0]);
    }
    const float nM = fmaxf(M, mx);
    if (nM != -INFINITY) {
      const float sc = M == -INFINITY ? 0.f : exp2f(M - nM);
      acc *= sc;
      den *= sc;
#pragma unroll
      for (int k = 0; k < kRound; ++k) {
        const int i = part * kRound + k;
        if (i < ns) {
          const float mi = s_ml[i][0];
          const float f = mi == -INFINITY ? 0.f : exp2f(mi - nM);
          acc = fmaf(f, ov[k], acc);
          den = fmaf(f, s_ml[i][1], den);
        }
      }
      M = nM;
    }
    __syncthreads();   // s_ml is refilled by the next round
  }
  s_part[part][0][c] = M;
  s_part[part][1][c] = den;
  s_part[part][2][c] = acc;
  __syncthreads();
  if (part == 0) {
    float nM = -INFINITY;
#pragma unroll
    for (int q = 0; q < NQ; ++q) nM = fmaxf(nM, s_part[q][0][c]);
    float o = 0.f;
    if (nM != -INFINITY) {
      float dd = 0.f, oo = 0.f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float Mq = s_part[q][0][c];
        const float f = Mq == -INFINITY ? 0.f : exp2f(Mq - nM);
        dd = fmaf(f, s_part[q][1][c], dd);
        oo = fmaf(f, s_part[q][2][c], oo);
      }
      o = dd > 0.f ? oo / dd : 0.f;
    }
    ocomb[c] = o;
  }
  __syncthreads();
  // o = R_V o' (row-major R_V: o_c = sum_j R_V[c][j] o'_j); thread (part, c)
  // sums its columns of row c, the parts meet in LDS.
  {
    const float* oc = &ocomb[kCols * part];
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < kCols / 4; ++j) {
      o = fmaf(r[j].x, oc[4 * j + 0], o);
      o = fmaf(r[j].y, oc[4 * j + 1], o);
      o = fmaf(r[j].z, oc[4 * j + 2], o);
      o = fmaf(r[j].w, oc[4 * j + 3], o);
    }
    red[part][c] = o;
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) o += red[q][tid];
    a.out[row_offset(a, b, h, g) + tid] = o;
  }
}

// Merge the 4 waves' states (see merge_wave_states) and store the
// work-group's partial in slot `part_slot` of the workspace.  Then take an
// arrival ticket of (b, h); the last of its n_parts work-groups combines the
// partials in slots [base_slot, base_slot + n_parts) and [tok_slot, tok_slot
// + n_tok) (the latter written by an earlier kernel), applies o = R_V o' and
// writes `out`.  ocomb: [GP][kHeadDim], s_m, s_l: [kCombineSlice][GP] LDS.
template <int GP>
__device__ void finish_work_group(const DecodeArgs& a, int b, int h, int64_t part_slot,
                                  int64_t base_slot, int n_parts, int64_t tok_slot, int n_tok,
                                  float (*wm)[GP], float (*wl)[GP], float (*wo)[GP][kHeadDim],
                                  float (*ocomb)[kHeadDim], float (*s_m)[GP], float (*s_l)[GP]) {
  const int G = a.group;
  const int tid = threadIdx.x;
  const int64_t head = int64_t(b) * a.n_kv_heads + h;
  float* part = a.partials + part_slot * G * kPartialStride;
  // Merged partial -> LDS (wo[0] is free once every thread has read its
  // inputs), then one wave stores it and takes the arrival ticket with an
  // agent-scope release (one per work-group).
  float* stage = &wo[0][0][0];
  merge_wave_states<GP>(G, wm, wl, wo, stage);
  __shared__ int is_last;
  if (tid < 64)
    for (int i = tid; i < G * kPartialStride; i += 64) store_agent(part + i, stage[i]);
  // (the barrier orders the other lanes' stores before thread 0's release)
  __syncthreads();
  if (tid == 0) {
    const int prev = fetch_add_acq_rel_agent(&a.tickets[head], 1);
    is_last = (prev == n_parts - 1);
  }
  __syncthreads();
  if (!is_last) return;
  // The last arriver's ticket acquired every other partial of (b, h); they
  // are read with agent-scope loads below.

  // Split weights f_i = 2^(m_i - M) / sum_k 2^(m_k - M) l_k, staged in LDS
  // in slices of kCombineSlice partials so that all loads of a slice are in
  // flight together.
  const int n_all = n_parts + n_tok;
  auto slot_ptr = [&](int i) -> const float* {
    const int64_t s = i < n_parts ? base_slot + i : tok_slot + (i - n_parts);
    return a.partials + s * G * kPartialStride;
  };
  __shared__ float s_M[GP], s_den[GP];
  const int wave = tid >> 6, lane = tid & 63;
  if (tid < GP) { s_M[tid] = -INFINITY; s_den[tid] = 0.f; }
  __syncthreads();
  for (int s0 = 0; s0 < n_all; s0 += kCombineSlice) {      // pass 1: M per head
    const int ns = min(kCombineSlice, n_all - s0);
    for (int i = tid; i < ns * G; i += blockDim.x)
      s_m[i / G][i % G] = load_agent(slot_ptr(s0 + i / G) + (i % G) * kPartialStride);
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
  for (int s0 = 0; s0 < n_all; s0 += kCombineSlice) {      // pass 2: weighted sums
    const int ns = min(kCombineSlice, n_all - s0);
    for (int i = tid; i < ns * G; i += blockDim.x) {
      const float* p = slot_ptr(s0 + i / G) + (i % G) * kPartialStride;
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
#pragma unroll 16
        for (int i = 0; i < ns; ++i)
          v = fmaf(s_m[i][g], load_agent(slot_ptr(s0 + i) + g * kPartialStride + 4 + c), v);
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
  // o = R_V o' (row-major R_V: o_i = sum_j R_V[i][j] o'_j).  Thread (half,
  // i) loads half of row i once (16 loads in flight) and applies it to every
  // head; the two halves meet in LDS (wo is free again).
  {
    const float* R = a.R_V + int64_t(h) * kHeadDim * kHeadDim;
    const int i = tid & (kHeadDim - 1), half = tid >> 7;
    const float4* row = reinterpret_cast<const float4*>(R + i * kHeadDim + 64 * half);
    float4 r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = row[j];
    float* red = &wo[0][0][0];   // [2][GP][kHeadDim]
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g < G) {
        const float* oc = &ocomb[g][64 * half];
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          o = fmaf(r[j].x, oc[4 * j + 0], o);
          o = fmaf(r[j].y, oc[4 * j + 1], o);
          o = fmaf(r[j].z, oc[4 * j + 2], o);
          o = fmaf(r[j].w, oc[4 * j + 3], o);
        }
        red[(half * GP + g) * kHeadDim + i] = o;
      }
    }
    __syncthreads();
    for (int k = tid; k < G * kHeadDim; k += blockDim.x) {
      const int g = k / kHeadDim, c = k % kHeadDim;
      a.out[row_offset(a, b, h, g) + c] =
          red[g * kHeadDim + c] + red[(GP + g) * kHeadDim + c];
    }
  }
  if (tid == 0) store_agent(&a.tickets[head], 0);   // ready for the next call on this workspace
}

}  // namespace kvq
