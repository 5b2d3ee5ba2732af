// Decode dispatch and pre-pass: fills the kernel arguments from the
// validated ABI structures, carves the caller's workspace (arrival counters,
// rotated queries, QK operands, range plan, split-K partials), launches the
// q-rotation / range-plan pre-pass (fused with the decode-step append for
// kvq_decode_step) and then the selected decode kernel.
#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>

#include "kvq2_append_common.h"
#include "kvq2_decode_common.h"

namespace kvq {

namespace {

// Threads of every pre-pass work-group (a constant: blockDim is an implicit
// kernel argument, and each read of one that missed the scalar cache cost
// the plan a memory latency).
constexpr int kPrePassThreads = 256;

// LDS of the range plan and of the q-rotation pre-pass.  The plan keeps
// W_b and the tile prefix of the first kPlanSeq sequences in LDS for the
// pair ranges (later sequences read them back from global memory).
constexpr int kPlanSeq = 1024;
struct PlanLds {
  int scan[256];
  int carry;
  int fbw[12];             // the range weights of this call: XCD [8], round [4]
  uint32_t fbraw[kFbWords];  // the self-calibration state as the previous call left it
  int rs[kChainGroups + 1];
  int w[kPlanSeq];         // W_b
  int pre[kPlanSeq];       // tile prefix before sequence b
};

// LDS of the plan's shared-prefix groups (prefix-aware decodes only).
constexpr int kPlanHash = 2 * kMaxPrefixMembers;   // open-addressing slots
struct GroupLds {
  int gs[kMaxPrefixGroups + 1];    // member starts (clamped)
  int gskip[kMaxPrefixGroups];     // whole prefix tiles
  int gvalid[kMaxPrefixGroups];    // some member is valid
  int grep[kMaxPrefixGroups];      // first valid member index, then its sequence
  int grs[kMaxPrefixGroups + 1];   // virtual tiles of earlier groups' items
  int gib[kMaxPrefixGroups + 1];   // first item
  int gw[kMaxPrefixGroups];        // virtual tiles per item
  int mseq[kMaxPrefixMembers];     // sequence of member m
  int mtiles[kMaxPrefixMembers];   // its whole INT2 tiles (-1: not a sequence)
  int mgroup[kMaxPrefixMembers];   // group of a valid member, else -1
  int slot[kPlanHash];             // sequence -> member index of its first listing
};

__device__ __forceinline__ uint32_t plan_hash(int b) {
  return (static_cast<uint32_t>(b) * 2654435761u) >> 21;   // 11 bits: kPlanHash slots
}
static_assert(kPlanHash == 2048, "plan_hash yields 11 bits");

// Member index of the first listing of sequence b, or -1.
__device__ __forceinline__ int first_listing(const GroupLds& L, int b) {
  uint32_t h = plan_hash(b);
  for (int k = 0; k < kPlanHash; ++k, h = (h + 1) & (kPlanHash - 1)) {
    const int m = L.slot[h];
    if (m < 0) return -1;
    if (L.mseq[m] == b) return m;
  }
  return -1;
}

// Tiles that sequence b's pieces skip (read by its group's row sets).
__device__ __forceinline__ int seq_skip_tiles(const GroupLds& L, int b) {
  const int m = first_listing(L, b);
  return m >= 0 && L.mgroup[m] >= 0 ? L.gskip[L.mgroup[m]] : 0;
}

// Shared-prefix groups, by the plan's work-group, in LDS: the valid members
// (a sequence's first listing, found through an open-addressing table keyed
// by sequence, whose whole INT2 tiles cover its group's prefix tiles), the
// tiles they skip, each group's row-set items (grp_info rows, with LDS
// copies for the cut) and the per-sequence tables of the later kernels.
template <int GP>
__device__ void plan_groups(const DecodeArgs& a, GroupLds& L) {
  constexpr int npt = chunks_per_tile(GP);
  const int tid = threadIdx.x, nt = kPrePassThreads;
  const int ngr = a.n_groups, B = a.batch, Hkv = a.n_kv_heads;
  const int cf = (a.n_sink + kChunkTokens - 1) / kChunkTokens;
  for (int g = tid; g <= ngr; g += nt) {
    L.gs[g] = a.member_start[g];
    if (g < ngr) {
      // tiles of the group's prefix: whole tiles from the first whole chunk
      const int pc = max(a.prefix_len[g], 0) / kChunkTokens;
      L.gskip[g] = pc > cf ? (pc - cf) / npt : 0;
      L.gvalid[g] = 0;
      L.grep[g] = INT_MAX;
    }
  }
  for (int m = tid; m < a.n_members; m += nt) L.mseq[m] = a.members[m];
  for (int h = tid; h < kPlanHash; h += nt) L.slot[h] = -1;
  __syncthreads();
  if (tid == 0) {   // member starts non-decreasing within [0, n_members]
    int prev = 0;
    for (int g = 0; g <= ngr; ++g) {
      prev = g == 0 ? 0 : min(max(L.gs[g], prev), a.n_members);
      L.gs[g] = prev;
    }
  }
  __syncthreads();
  const int nm = L.gs[ngr];
  // first listing of every sequence: the table keeps the smallest member
  // index per sequence (a slot, once claimed, only ever holds that sequence)
  for (int m = tid; m < nm; m += nt) {
    const int b = L.mseq[m];
    int tiles = -1;
    if (b >= 0 && b < B) {
      const Int2Range rg = int2_range(a, a.seq_len[b], npt);
      tiles = (rg.cl - rg.cf) / npt;
      uint32_t h = plan_hash(b);
      for (int k = 0; k < kPlanHash; ++k, h = (h + 1) & (kPlanHash - 1)) {
        int cur = L.slot[h];
        if (cur < 0) {
          cur = atomicCAS(&L.slot[h], -1, m);
          if (cur < 0) break;
        }
        if (L.mseq[cur] == b) {
          atomicMin(&L.slot[h], m);
          break;
        }
      }
    }
    L.mtiles[m] = tiles;
  }
  __syncthreads();
  for (int m = tid; m < nm; m += nt) {
    const int b = L.mseq[m];
    int grp = -1;
    if (L.mtiles[m] >= 0 && first_listing(L, b) == m) {
      int lo = 0, hi = ngr;   // group of m: the largest g with gs[g] <= m
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (L.gs[mid] <= m) lo = mid; else hi = mid;
      }
      const int skip = L.gskip[lo];
      if (skip > 0 && L.mtiles[m] >= skip) {
        grp = lo;
        atomicMin(&L.grep[lo], m);
        L.gvalid[lo] = 1;
      }
    }
    L.mgroup[m] = grp;
  }
  __syncthreads();
  for (int g = tid; g < ngr; g += nt) L.grep[g] = L.gvalid[g] ? L.mseq[L.grep[g]] : 0;
  __syncthreads();
  if (tid == 0) {
    int rs = 0, ib = 0;
    for (int g = 0; g < ngr; ++g) {
      const int rows = (L.gs[g + 1] - L.gs[g] + 3) / 4;
      const int skip = L.gvalid[g] ? L.gskip[g] : 0;
      const int w = max(1, a.rs_cost * skip) + a.piece_cost;
      L.grs[g] = rs;
      L.gib[g] = ib;
      L.gw[g] = w;
      int32_t* gi = a.grp_info + g * kGrpInfo;
      gi[kGiRsPrefix] = rs;
      gi[kGiWidth] = w;
      gi[kGiSkip] = skip;
      gi[kGiRep] = L.grep[g];
      gi[kGiRowSets] = rows;
      gi[kGiItemBase] = ib;
      gi[kGiMemberStart] = L.gs[g];
      gi[kGiMemberEnd] = L.gs[g + 1];
      rs += Hkv * rows * w;
      ib += Hkv * rows;
    }
    L.grs[ngr] = rs;
    L.gib[ngr] = ib;
  }
  // per-sequence tables of the stream and combine kernels (read after this
  // launch)
  for (int b = tid; b < B; b += nt) {
    const int m = first_listing(L, b);
    const int grp = m >= 0 ? L.mgroup[m] : -1;
    a.seq_member[b] = m;
    a.seq_group[b] = grp;
    a.seq_skip[b] = grp >= 0 ? L.gskip[grp] : 0;
  }
  __syncthreads();
}

template <int KG>
struct PrologueLds {
  float qs[KG][kHeadDim];           // q, then q'
  float buf[2 * KG * kHeadDim];     // rotation half sums [2][KG][128]
  float qsum[KG];
  int qexp[KG];
};

// One step of the self-calibrating range weights, by the 64 lanes of one
// wave (lane c < 32 holds cell (round c / 8, XCD c % 8)): the mean duration
// of the ranges of each XCD (and of each dispatch round) measured by the
// previous call with this state, against the mean of all, scales that XCD's
// (round's) weight by sqrt(mean / its mean); the weights are then
// renormalised to a mean of 1024 and clamped to [724, 1448] (each within a
// factor of two of every other, so that no weighted range is empty) and
// stored; the caller clears the sums.  Before the first measurement, and
// while the ranges last under 50 us, the launch's weights stand.  fb_in:
// the state as read at the plan's start (LDS); fb: the state itself; w
// (LDS): XCD weights [8], round weights [4], the launch's on entry and this
// call's on return.
__device__ void feedback_update(const uint32_t* fb_in, uint32_t* fb, int rounds, int* w) {
  const int c = threadIdx.x & 63, r = (c >> 3) & 3, x = c & 7;
  const bool init = fb_in[kFbXw] != 0;
  // this lane's cell, and the current weights of its XCD and round
  const bool cell = c < 32 && r < rounds;
  const float v = cell ? static_cast<float>(fb_in[kFbSum + c]) : 0.f;
  const float k = cell ? static_cast<float>(fb_in[kFbCnt + c]) : 0.f;
  const int lx = w[x], lr = w[8 + r];   // the launch's
  int wx = init ? static_cast<int>(fb_in[kFbXw + x]) : lx;
  int wr = init ? static_cast<int>(fb_in[kFbRw + r]) : lr;
  const float s = wave_sum(v), n = wave_sum(k);
  // per XCD: the lanes c ^ 8, c ^ 16; per round: c ^ 1, c ^ 2, c ^ 4
  float sx = v + __shfl_xor(v, 8), nx = k + __shfl_xor(k, 8);
  sx += __shfl_xor(sx, 16);
  nx += __shfl_xor(nx, 16);
  float sr = v + __shfl_xor(v, 1), nr = k + __shfl_xor(k, 1);
  sr += __shfl_xor(sr, 2);
  nr += __shfl_xor(nr, 2);
  sr += __shfl_xor(sr, 4);
  nr += __shfl_xor(nr, 4);
  // Ranges shorter than kFbMinTicks (batch-1 decodes) are dominated by
  // fixed latencies, not by their share of the tiles: the launch weights.
  constexpr float kFbMinTicks = 5000.f;   // 50 us of the 100 MHz clock
  if (n > 0.f && s < kFbMinTicks * n) {
    wx = lx;
    wr = lr;
  }
  // every XCD and every used round measured
  const bool have = c < 32 && nx > 0.f && (r >= rounds || nr > 0.f);
  const bool every = n > 0.f && s >= kFbMinTicks * n &&
                     __builtin_amdgcn_ballot_w64(c < 32 && !have) == 0;
  if (every) {
    const float mean = s / n;
    const float fx = sqrtf(mean * nx / sx);
    const float fr = r < rounds ? sqrtf(mean * nr / sr) : 1.f;
    // renormalise: the mean of the new XCD weights (lanes 0 .. 7) and of the
    // used rounds' (lanes 0, 8, 16, 24 below rounds) is 1024
    const float mx = wave_sum(c < 8 ? wx * fx : 0.f) / 8.f;
    const float mr = wave_sum(c < 32 && x == 0 && r < rounds ? wr * fr : 0.f) /
                     static_cast<float>(rounds);
    wx = min(1448, max(724, static_cast<int>(wx * fx * 1024.f / mx + 0.5f)));
    if (r < rounds) wr = min(1448, max(724, static_cast<int>(wr * fr * 1024.f / mr + 0.5f)));
  }
  __builtin_amdgcn_wave_barrier();   // (every lane has read w)
  if (c < 8) {
    fb[kFbXw + c] = static_cast<uint32_t>(wx);
    w[c] = wx;
  }
  if (c < 32 && x == 0) {   // lane 8 r holds round r's weight
    fb[kFbRw + r] = static_cast<uint32_t>(wr);
    w[8 + r] = wr;
  }
}

// The equal-range plan of the MFMA decode, by one work-group of 256 threads
// (PRE: with shared-prefix groups, whose LDS is *L).
template <int GP, bool PRE = false>
__device__ void plan_ranges(const DecodeArgs& a, PlanLds& P, GroupLds* L = nullptr) {
  constexpr int npt = chunks_per_tile(GP);
  const int tid = threadIdx.x;
  // Every argument the plan reads is loaded here, in one batch of scalar
  // loads waited for once: fetched where each is first used, the argument
  // block's cache lines missed one after another, a memory latency each.
  {
    int v[13] = {a.batch, a.n_sink, a.n_recent, a.piece_cost, a.chain_groups, a.n_kv_heads,
                 a.round_size, a.round_weight[0], a.round_weight[1], a.round_weight[2],
                 a.round_weight[3], a.xcd_weight[0], a.xcd_weight[7]};
#pragma unroll
    for (int k = 0; k < 13; ++k) asm volatile("" : : "s"(v[k]));
    const void* ptr[4] = {a.seq_len, a.tile_prefix, a.range_start, a.pair_range};
#pragma unroll
    for (int k = 0; k < 4; ++k) asm volatile("" : : "s"(ptr[k]));
  }
  // W_b = max(1, whole INT2 tiles of sequence b) + piece_cost;
  // tile_prefix[b] = W_0 + ... + W_{b-1} (inclusive Hillis-Steele scan
  // over blocks of 256 sequences).
  int* scan = P.scan;
  int& carry = P.carry;
  // the self-calibration state, read now so that its latency overlaps the
  // scan's (the scan's barriers publish it)
  if (a.feedback != nullptr && tid < kFbWords) P.fbraw[tid] = a.feedback[tid];
  if constexpr (PRE) plan_groups<GP>(a, *L);
  if (tid == 0) { carry = 0; a.tile_prefix[0] = 0; }
  __syncthreads();
  for (int base = 0; base < a.batch; base += 256) {
    const int bb = base + tid;
    int w = 0;
    if (bb < a.batch) {
      const Int2Range rg = int2_range(a, a.seq_len[bb], npt);
      int skip = 0;
      if constexpr (PRE) skip = seq_skip_tiles(*L, bb);
      w = max(1, (rg.cl - rg.cf) / npt - skip) + a.piece_cost;
    }
    scan[tid] = w;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int v = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (bb < a.batch) a.tile_prefix[bb + 1] = carry + scan[tid];
    if (bb < a.batch && bb < kPlanSeq) {
      P.w[bb] = w;
      P.pre[bb] = carry + scan[tid] - w;
    }
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  // The cut into chain_groups ranges (weighted by dispatch round when
  // every range keeps at least a few tiles, else equal), then the first
  // and last range of every (b, h).
  int* rs = P.rs;
  const int nwg = a.chain_groups;
  const int Hkv = a.n_kv_heads;
  // the (b, h) pieces, then the row-set items of shared-prefix groups
  const int64_t pairs_total = int64_t(Hkv) * carry;
  int64_t total = pairs_total;
  if constexpr (PRE) total += L->grs[a.n_groups];
  const int rsz = a.round_size, rounds = rsz > 0 ? nwg / rsz : 0;
  const bool weighted = rsz > 0 && rsz % 8 == 0 && rounds >= 2 && rounds <= 4 &&
                        rounds * rsz == nwg && total >= 4 * int64_t(nwg);
  // Work-group j weighs round_weight[j / rsz] * xcd_weight[j % 8]; range i
  // starts at total * (weight of work-groups < i) / (weight of all).  A round
  // (rsz, a multiple of 8 when weighted) holds every XCD rsz / 8 times.
  // Each thread's cut is a closed form in 32-bit integers and fp64 (exact:
  // every weight sum stays below 2^53) on weights held in registers: 64-bit
  // integer products and divisions per range made this loop the longest part
  // of the pre-pass, and so did reading the weights from the argument block.
  int xw[8], rw[4];
#pragma unroll
  for (int x = 0; x < 8; ++x) xw[x] = a.xcd_weight[x];
#pragma unroll
  for (int r = 0; r < 4; ++r) rw[r] = a.round_weight[r];
  if (a.feedback != nullptr && weighted) {
    if (tid == 0) {
#pragma unroll
      for (int x = 0; x < 8; ++x) P.fbw[x] = xw[x];
#pragma unroll
      for (int r = 0; r < 4; ++r) P.fbw[8 + r] = rw[r];
    }
    __syncthreads();
    if (tid < 64) {
      feedback_update(P.fbraw, a.feedback, rounds, P.fbw);
      a.feedback[kFbSum + tid] = 0u;   // sums and counts, for this call's ranges
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 8; ++x) xw[x] = P.fbw[x];
#pragma unroll
    for (int r = 0; r < 4; ++r) rw[r] = P.fbw[8 + r];
  }
  int xsum = 0;
#pragma unroll
  for (int x = 0; x < 8; ++x) xsum += xw[x];
  // weight of the first k work-groups of one round, over its xcd weights
  auto xcd_prefix = [&](int k) {
    int c = (k >> 3) * xsum;
    const int m = k & 7;
#pragma unroll
    for (int x = 0; x < 7; ++x) c += x < m ? xw[x] : 0;
    return c;
  };
  const double round_w = xcd_prefix(rsz);   // xcd weight of one whole round
  double ctot = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < rounds) ctot += double(rw[r]) * round_w;
  const int64_t q = (total + nwg - 1) / nwg;
  // total * c / ctot: monotone in c, truncated, and range nwg ends exactly
  // at total (total < 2^31: range starts are 32-bit)
  const double scale = double(total) / (ctot > 0 ? ctot : 1.0);
  const double dtotal = double(total);
  for (int i = tid; i <= nwg; i += kPrePassThreads) {
    int v;
    if (!weighted) {
      v = static_cast<int>(min(total, int64_t(i) * q));
    } else {
      const int r0 = min(i / rsz, rounds);   // i's round (rounds at i == nwg)
      double c = 0;   // whole rounds before r0
#pragma unroll
      for (int r = 0; r < 4; ++r) c += r < r0 ? double(rw[r]) * round_w : 0.0;
      const int rw0 = r0 == 0 ? rw[0] : r0 == 1 ? rw[1] : r0 == 2 ? rw[2] : r0 == 3 ? rw[3] : 0;
      c += double(rw0) * double(xcd_prefix(i - r0 * rsz));
      v = i == nwg ? static_cast<int>(total) : static_cast<int>(fmin(dtotal, trunc(c * scale)));
    }
    rs[i] = v;
    a.range_start[i] = v;
  }
  __syncthreads();
  // (largest i < nwg with rs[i] <= x0) | (the same for x1) << 16: both
  // searches in one loop of power-of-two steps, so that their dependent LDS
  // reads overlap (rs[0] = 0 <= x)
  int top = 1;
  while (2 * top < nwg) top *= 2;
  auto range_pair = [&](int x0, int x1) {
    int i0 = 0, i1 = 0;
    for (int st = top; st > 0; st >>= 1) {
      const int j0 = min(i0 + st, nwg - 1), j1 = min(i1 + st, nwg - 1);
      const int r0 = rs[j0], r1 = rs[j1];
      if (r0 <= x0) i0 = j0;
      if (r1 <= x1) i1 = j1;
    }
    return i0 | (i1 << 16);
  };
  for (int pr = tid; pr < a.batch * Hkv; pr += kPrePassThreads) {
    const int bb = pr / Hkv, hh = pr % Hkv;
    int wbb, pre_b;
    if (bb < kPlanSeq) {
      wbb = P.w[bb];
      pre_b = P.pre[bb];
    } else {   // recomputed, and the prefix read back from the scan output
      const Int2Range rg = int2_range(a, a.seq_len[bb], npt);
      int skip = 0;
      if constexpr (PRE) skip = seq_skip_tiles(*L, bb);
      wbb = max(1, (rg.cl - rg.cf) / npt - skip) + a.piece_cost;
      pre_b = a.tile_prefix[bb];
    }
    const int sp = Hkv * pre_b + hh * wbb;
    a.pair_range[pr] = range_pair(sp, sp + wbb - 1);
  }
  // first and last range of every row-set item
  if constexpr (PRE) {
    const int ngr = a.n_groups;
    for (int q = tid; q < L->gib[ngr]; q += kPrePassThreads) {
      int lo = 0, hi = ngr;   // group of item q: the largest g with gib[g] <= q
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (L->gib[mid] <= q) lo = mid; else hi = mid;
      }
      const int64_t sq = pairs_total + L->grs[lo] + int64_t(q - L->gib[lo]) * L->gw[lo];
      a.item_range[q] = range_pair(static_cast<int>(sq), static_cast<int>(sq + L->gw[lo] - 1));
    }
  }
}

// Pre-pass of the decode, one work-group per (KV head h, sequence b):
//  * q'[g] = alpha R_K[h]^T q[b][hG+g] (OSCAR summary sec. 2.2-B: the query
//    is rotated once instead of un-rotating every cached key), sum(q'[g])
//    and the exponent e with 2^-e max|q'[g]| < 1, stored for the later
//    kernels and, for the MFMA decode, its QK operand block;
//  * MFMA decode: one more work-group, (Hkv, 0), computes the plan of the
//    equal-range decode alongside the others (the rest of column Hkv exits
//    at once).
// GP: MFMA head-group width (2, 4 or 8); 0 for the VALU decode.
// Work-group (hx, b) of the pre-pass grid (Hkv + 1, B) (Hkv, B for the
// VALU decode), with its LDS.
template <int GP, bool PRE = false>
__device__ __forceinline__ void prologue_block(const DecodeArgs& a, int hx, int b,
                                               PrologueLds<(GP > 0 ? GP : kMaxGroup)>& Lq,
                                               PlanLds& P, GroupLds* L = nullptr) {
  constexpr int KG = GP > 0 ? GP : kMaxGroup;   // query heads per KV head held
  if constexpr (GP > 0) {
    if (hx == a.n_kv_heads) {
      if (b == 0) plan_ranges<GP, PRE>(a, P, L);
      return;
    }
  }
  float (*qs)[kHeadDim] = Lq.qs;
  float* buf = Lq.buf;
  float* qsum = Lq.qsum;
  int* qexp = Lq.qexp;
  const int h = hx;
  const int G = a.group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float (*part)[KG][kHeadDim] = reinterpret_cast<float (*)[KG][kHeadDim]>(buf);
  // q of the group's heads; rows g >= G are zero (they take part in the
  // rotation below without branches)
#pragma unroll
  for (int k = 0; k < KG * kHeadDim / 256; ++k) {
    const int i = tid + 256 * k, g = i / kHeadDim, c = i % kHeadDim;
    qs[g][c] = g < G ? bf16_bits_to_float(
                           a.q[row_offset(a, b, h, g) + c])
                     : 0.f;
  }
  __syncthreads();
  // Thread (half, c) sums j in [64 half, 64 half + 64) for every head of the
  // group: one coalesced load of R row j feeds KG independent FMA chains.
  const float* R = a.R_K + int64_t(h) * kHeadDim * kHeadDim;
  {
    const int c = tid & (kHeadDim - 1), half = tid >> 7;
    float acc[KG];
#pragma unroll
    for (int g = 0; g < KG; ++g) acc[g] = 0.0f;
    const int j0 = 64 * half;
    float r[64];   // all 64 loads in flight together
#pragma unroll
    for (int u = 0; u < 64; ++u) r[u] = R[(j0 + u) * kHeadDim + c];
    // (empty asm: one wait for all 64 loads instead of a schedule in batches)
#pragma unroll
    for (int u = 0; u < 64; u += 4) asm volatile("" : "+v"(r[u]), "+v"(r[u + 1]), "+v"(r[u + 2]), "+v"(r[u + 3]));
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      if (GP == 0 && g >= G) break;   // (uniform) the VALU layout holds up to 16 heads
      const float4* qv = reinterpret_cast<const float4*>(&qs[g][j0]);
#pragma unroll
      for (int u4 = 0; u4 < 16; ++u4) {
        const float4 x = qv[u4];
        acc[g] = fmaf(r[4 * u4 + 0], x.x, acc[g]);
        acc[g] = fmaf(r[4 * u4 + 1], x.y, acc[g]);
        acc[g] = fmaf(r[4 * u4 + 2], x.z, acc[g]);
        acc[g] = fmaf(r[4 * u4 + 3], x.w, acc[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < KG; ++g) part[half][g][c] = acc[g];
  }
  __syncthreads();
  float* dst = a.qrot + qrot_offset(a, b, h);
  for (int i = tid; i < G * kHeadDim; i += kPrePassThreads) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    const float v = (part[0][g][c] + part[1][g][c]) * a.alpha;
    qs[g][c] = v;
    dst[g * kQStride + c] = v;
  }
  __syncthreads();
  for (int g = wave; g < G; g += kPrePassThreads / 64) {
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
  if constexpr (GP > 0) {
    // QK operand of the MFMA kernel in its per-lane layout: lane (gq, n)
    // holds column n = 2GP blk + GP t + g (t = 0: f16 hi part, 1: lo part of
    // q'[g] scaled by 2^-e_g 2^(8 - 2s)) for the 32 k-slots of its lane group.
    // With one (scale, zero) pair per vector every column block holds all
    // channels.  With ng quantization groups, block blk holds only the
    // channels of the groups k with k mod nb = blk mod nb, nb = min(ng,
    // nblk) (zero elsewhere), so that each block's dot is one group's; when
    // the tile has fewer blocks than groups, the kernel runs one product per
    // set c of nblk groups with the code operand restricted to that set's
    // groups, and block blk of set c is group c nblk + blk.
    constexpr int NBLK = 16 / (2 * GP);
    const int ng = a.ng;
    const int sets = (GP <= 4 && ng > NBLK) ? ng / NBLK : 1;
    const int nb = ng < NBLK ? ng : NBLK;
    const int gch = kHeadDim / ng;            // channels per group
    // sums of q'[g] over each 32-channel quarter (ng <= 4 groups are unions)
    __shared__ float qq4[GP > 0 ? GP : 1][4];
    if (tid < G * 4) {
      const int g = tid >> 2, k = tid & 3;
      float sum = 0.f;
      for (int c = 0; c < 32; ++c) sum += qs[g][32 * k + c];
      qq4[g][k] = sum;
    }
    __syncthreads();
    uint32_t* bq = a.bq + (int64_t(b) * a.n_kv_heads + h) * kBqWords;
    const int kk = tid >> 6;                 // 4 k-steps x 64 lanes
    const int gq = lane >> 4, n = lane & 15;
    const int blk = n / (2 * GP), j = n % (2 * GP), g = j % GP;
    const bool hi_col = j < GP, ok = g < G;
    const float down = ok ? ldexpf(1.0f, -qexp[g]) : 0.f;
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
      for (int e = 0; e < 2; ++e) {
        int ch, sc;
        kslot_channel(gq, kk, 2 * q + e, ch, sc);
        const bool in = ng == 1 || (ch / gch) % nb == blk % nb;
        const float v = (ok && in) ? qs[g][ch] * down * ldexpf(1.0f, 8 - 2 * sc) : 0.f;
        const _Float16 vh = static_cast<_Float16>(v);
        const _Float16 vl = static_cast<_Float16>(v - static_cast<float>(vh));
        const uint32_t bits = __builtin_bit_cast(uint16_t, hi_col ? vh : vl);
        word |= bits << (16 * e);
      }
      bq[lane * 16 + kk * 4 + q] = word;
    }
    if (kk == 0) {
      const float qscale = ok ? ldexpf(1.0f, 16 + qexp[g]) : 1.0f;
      float* lc = reinterpret_cast<float*>(bq) + kBqOperandWords + 4 * lane;
      lc[0] = qscale;
      for (int c = 0; c < 2; ++c) {
        float qbar = ok ? qsum[g] : 0.f;
        if (ng > 1 && ok && c < sets) {
          const int grp = (c * NBLK + blk) % ng;
          qbar = 0.f;
          for (int k = 0; k < 4; ++k)
            if ((32 * k) / gch == grp) qbar += qq4[g][k];
        }
        lc[1 + c] = qbar / qscale;
      }
      lc[3] = 0.f;
    }
  }
}

template <int GP>
__global__ __launch_bounds__(256, 5) void prologue_kernel(DecodeArgs a) {
  __shared__ PrologueLds<(GP > 0 ? GP : kMaxGroup)> Lq;
  __shared__ PlanLds P;
  prologue_block<GP>(a, blockIdx.x, blockIdx.y, Lq, P);
}

// The pre-pass of a decode with shared-prefix groups (MFMA decode): the
// plan also resolves the groups (GroupLds).
template <int GP>
__global__ __launch_bounds__(256) void prologue_prefix_kernel(DecodeArgs a) {
  __shared__ PrologueLds<GP> Lq;
  __shared__ PlanLds P;
  __shared__ GroupLds L;
  prologue_block<GP, true>(a, blockIdx.x, blockIdx.y, Lq, P, &L);
}

// The pre-pass of a fused decode step: the work-groups of the decode-step
// append (grid (n_app_x, Hkv, 2), first) and those of the q-rotation
// pre-pass (grid (Hkv + 1, B)) in one launch.  They are independent: the
// append writes the cache, the pre-pass reads only q, R_K and the lengths.
// One LDS arena serves either role.
template <int GP>
__global__ __launch_bounds__(256) void step_prologue_kernel(AppendArgs aa, DecodeArgs a,
                                                            int n_app_x) {
  constexpr size_t kAppendLds =
      sizeof(float) * kHeadDim * kHeadDim + sizeof(double) * kWaves * kHeadDim;
  constexpr size_t kPreLds = sizeof(PrologueLds<GP>) + sizeof(PlanLds);
  __shared__ __attribute__((aligned(16))) unsigned char arena[kAppendLds > kPreLds ? kAppendLds
                                                                                     : kPreLds];
  const int x = blockIdx.x;
  const int n_app = n_app_x * a.n_kv_heads * 2;
  if (x < n_app) {
    const int bx = x % n_app_x, h = (x / n_app_x) % a.n_kv_heads;
    const int kind = x / (n_app_x * a.n_kv_heads);
    append_step_block(aa, bx, h, kind, reinterpret_cast<float*>(arena),
                      reinterpret_cast<double (*)[kHeadDim]>(
                          arena + sizeof(float) * kHeadDim * kHeadDim));
    return;
  }
  const int y = x - n_app, H1 = a.n_kv_heads + 1;
  prologue_block<GP>(a, y % H1, y / H1, *reinterpret_cast<PrologueLds<GP>*>(arena),
                     *reinterpret_cast<PlanLds*>(arena + sizeof(PrologueLds<GP>)));
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = 0u;
}

// The decode workspace of kvq_decode_attention_noalloc: one copy per GPU,
// held from the first load of the library on that GPU until the process
// ends.  Host code never uses this name as an address: its device address
// comes from hipGetSymbolAddress, once per device (static_scratch).
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// The self-calibrating range-weight states of this GPU (kFb* layout), zero
// when the library is loaded; addressed like scratch (decode_feedback).
__device__ __align__(256) uint32_t feedback_state[kFbStates * kFbWords];

}  // namespace

int static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices];
  static int status[kMaxDevices];
  static std::once_flag once[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::call_once(once[dev], [dev] {
    // runs with device `dev` current (the caller's current device)
    status[dev] = static_cast<int>(hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)));
  });
  if (status[dev] != 0) return status[dev];
  *ptr = addr[dev];
  return 0;
}

int decode_feedback(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices];
  static int status[kMaxDevices];
  static std::once_flag once[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::call_once(once[dev], [dev] {
    status[dev] = static_cast<int>(hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(feedback_state)));
  });
  if (status[dev] != 0) return status[dev];
  *ptr = addr[dev];
  return 0;
}

int launch_zero_words(void* p, size_t bytes, void* stream) {
  const size_t n = bytes / 4;
  if (n == 0) return 0;
  const unsigned grid = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(p), n);
  return static_cast<int>(hipGetLastError());
}

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);
void set_chain_geometry(DecodeArgs& a, int batch, int max_seq_len);
int launch_decode_mfma(const DecodeArgs& a, int batch, int max_seq_len, void* stream);

namespace {

DecodeArgs make_decode_args(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                            const kvq_cache& cache, int32_t batch, const int32_t* seq_len,
                            const uint16_t* q, float* out, void* workspace,
                            const DecodePlan& plan, DecodeKernel which, int32_t n_query,
                            int32_t query_base, int32_t query_count,
                            const kvq_prefix_groups* groups) {
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
  a.head_group = d.n_q_heads / d.n_kv_heads;
  a.n_query = n_query;
  a.query_base = query_base;
  a.query_count = query_count;
  a.group = a.head_group * n_query;
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
  a.ng = d.quant_group == 0 ? 1 : kHeadDim / d.quant_group;
  a.chunk_bytes = chunk_bytes_for(a.ng);
  a.page_bytes = int64_t(d.n_kv_heads) * cpp * a.chunk_bytes;
  a.seq_len = seq_len;
  a.q = q;
  a.out = out;
  a.tickets = static_cast<int32_t*>(workspace);
  a.batch = batch;
  char* ws = static_cast<char*>(workspace);
  a.qrot = reinterpret_cast<float*>(ws + plan.ticket_bytes);
  a.bq = reinterpret_cast<uint32_t*>(ws + plan.ticket_bytes + plan.qrot_bytes);
  a.tile_prefix = reinterpret_cast<int32_t*>(ws + plan.ticket_bytes + plan.qrot_bytes + plan.bq_bytes);
  {
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    char* pre = reinterpret_cast<char*>(a.tile_prefix);
    a.range_start = reinterpret_cast<int32_t*>(pre + r256((size_t(batch) + 1) * sizeof(int32_t)));
    a.pair_range = reinterpret_cast<int32_t*>(pre + r256((size_t(batch) + 1) * sizeof(int32_t)) +
                                              r256((size_t(kChainGroups) + 1) * sizeof(int32_t)));
  }
  char* grp = ws + plan.ticket_bytes + plan.qrot_bytes + plan.bq_bytes + plan.prefix_bytes;
  a.partials = reinterpret_cast<float*>(grp + plan.group_bytes);
  if (plan.n_groups > 0 && groups != nullptr) {
    auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t bb = r256(size_t(batch) * sizeof(int32_t));
    a.n_groups = plan.n_groups;
    a.n_members = plan.n_members;
    a.rs_cost = plan.rs_cost;
    a.member_start = groups->member_start;
    a.members = groups->members;
    a.prefix_len = groups->prefix_len;
    a.seq_skip = reinterpret_cast<int32_t*>(grp);
    a.seq_member = reinterpret_cast<int32_t*>(grp + bb);
    a.seq_group = reinterpret_cast<int32_t*>(grp + 2 * bb);
    a.grp_info = reinterpret_cast<int32_t*>(grp + 3 * bb);
    a.item_range = reinterpret_cast<int32_t*>(
        grp + 3 * bb + r256(size_t(plan.n_groups) * kGrpInfo * sizeof(int32_t)));
    a.rs_slot0 = plan.rs_slot0;
  }
  const int G = a.group;
  // the matrix-core kernel takes narrower quantization groups for up to four
  // rows per (b, h)
  a.gp = (which == kDecodeValu || G > 8 || (a.ng != 1 && G > 4)) ? 0
                                                                : (G <= 2 ? 2 : G <= 4 ? 4 : 8);
  a.n_split_int2 = plan.n_split_int2;
  a.n_split = plan.n_split;
  a.piece_cost = plan.piece_cost;
  a.n_tok_slices = plan.n_tok_slices;
  a.tok_slot0 = plan.tok_slot0;
  return a;
}

// The self-calibrating weight state of a launch: one per (G <= 4 or G = 8,
// 2 .. 4 dispatch rounds); none when the cut is not weighted, when ranges
// hold fewer than kFbMinTiles tiles (fixed latencies, not the weights, set
// their durations; measured at one sequence of 131072 tokens the state's
// bookkeeping only lengthened the pre-pass by ~3 us) or with KVQ_ADAPT=0.
constexpr int64_t kFbMinTiles = 128;
int attach_feedback(DecodeArgs& a, int batch, int max_seq_len) {
  a.feedback = nullptr;
  if (!decode_tuning().adapt || a.round_size <= 0) return 0;
  const int rounds = a.chain_groups / a.round_size;
  if (rounds < 2 || rounds > 4 || rounds * a.round_size != a.chain_groups ||
      a.round_size % 8 != 0)
    return 0;
  const int64_t int2_end = std::max<int64_t>(a.n_sink, int64_t(max_seq_len) - a.n_recent);
  const int64_t tiles = int64_t(batch) * a.n_kv_heads *
                        ((int2_end / kChunkTokens) / chunks_per_tile(a.gp));
  if (tiles < kFbMinTiles * a.chain_groups) return 0;
  void* base = nullptr;
  const int err = decode_feedback(&base);
  if (err != 0) return err;
  a.feedback = static_cast<uint32_t*>(base) + ((a.group > 4 ? 3 : 0) + rounds - 2) * kFbWords;
  return 0;
}

}  // namespace

int launch_decode(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                  const kvq_cache& cache, int32_t batch, const int32_t* seq_len,
                  int32_t max_seq_len, const uint16_t* q, float* out, void* workspace,
                  const DecodePlan& plan, DecodeKernel which, void* stream, int32_t n_query,
                  int32_t query_base, int32_t query_count, const kvq_prefix_groups* groups) {
  DecodeArgs a = make_decode_args(d, sm_scale, layer, cache, batch, seq_len, q, out, workspace,
                                  plan, which, n_query, query_base, query_count, groups);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.gp != 0) {
    set_chain_geometry(a, batch, max_seq_len);
    const int err = attach_feedback(a, batch, max_seq_len);
    if (err != 0) return err;
  }
  const dim3 pgrid(d.n_kv_heads + (a.gp != 0 ? 1 : 0), batch);
  if (a.n_groups > 0) {
    if (a.gp == 2) hipLaunchKernelGGL(prologue_prefix_kernel<2>, pgrid, dim3(256), 0, st, a);
    else if (a.gp == 4) hipLaunchKernelGGL(prologue_prefix_kernel<4>, pgrid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(prologue_prefix_kernel<8>, pgrid, dim3(256), 0, st, a);
  } else if (a.gp == 2) hipLaunchKernelGGL(prologue_kernel<2>, pgrid, dim3(256), 0, st, a);
  else if (a.gp == 4) hipLaunchKernelGGL(prologue_kernel<4>, pgrid, dim3(256), 0, st, a);
  else if (a.gp == 8) hipLaunchKernelGGL(prologue_kernel<8>, pgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(prologue_kernel<0>, pgrid, dim3(256), 0, st, a);
  const int err = static_cast<int>(hipGetLastError());
  if (err != 0) return err;
  if (a.gp == 0) return launch_decode_valu(a, batch, stream);
  return launch_decode_mfma(a, batch, max_seq_len, stream);
}


int launch_decode_step(const kvq_dims& d, float sm_scale, const kvq_layer& layer,
                       const kvq_cache& cache, int32_t batch, const int32_t* start_pos,
                       const int32_t* cu_new, int32_t total_new, const uint16_t* k_new,
                       const uint16_t* v_new, const int32_t* seq_len, int32_t max_seq_len,
                       const uint16_t* q, float* out, void* workspace, const DecodePlan& plan,
                       void* stream) {
  DecodeArgs a = make_decode_args(d, sm_scale, layer, cache, batch, seq_len, q, out, workspace,
                                  plan, kDecodeMfma, 1, 0, 1, nullptr);
  const AppendArgs aa = make_append_args(d, layer, cache, batch, start_pos, cu_new, total_new,
                                         k_new, v_new);
  if (a.gp == 0 || aa.tokens_per_block != kWaves) return -1;   // not a fused-step shape
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_chain_geometry(a, batch, max_seq_len);
  {
    const int err = attach_feedback(a, batch, max_seq_len);
    if (err != 0) return err;
  }
  const int n_app_x = (total_new + kWaves - 1) / kWaves;
  const dim3 grid(n_app_x * d.n_kv_heads * 2 + (d.n_kv_heads + 1) * batch);
  if (a.gp == 2) hipLaunchKernelGGL(step_prologue_kernel<2>, grid, dim3(256), 0, st, aa, a, n_app_x);
  else if (a.gp == 4) hipLaunchKernelGGL(step_prologue_kernel<4>, grid, dim3(256), 0, st, aa, a, n_app_x);
  else hipLaunchKernelGGL(step_prologue_kernel<8>, grid, dim3(256), 0, st, aa, a, n_app_x);
  const int err = static_cast<int>(hipGetLastError());
  if (err != 0) return err;
  return launch_decode_mfma(a, batch, max_seq_len, stream);
}

}  // namespace kvq
