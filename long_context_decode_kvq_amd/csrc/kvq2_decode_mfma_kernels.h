// Split-K decode attention on the matrix cores (gfx950 MFMA, f16 in, fp32
// accumulate).  OSCAR technical summary, sec. 2.2-B: the fused kernel
// unpacks and dequantizes INT2 history in registers and attends over it.
//
// Why MFMA: at INT2 one HBM byte carries 14 (G = 4) to 28 (G = 8) useful
// multiply-adds, beyond what fp32 VALU sustains at HBM speed.  Both products
// of a 16-token chunk are small dense contractions:
//   QK:  S^T[token][col] = sum_ch codes[token][ch] * Bq[ch][col]
//        (16x16x32 f16, four k-steps cover the 128 channels)
//   PV:  O[row][ch]     += sum_tok W[row][tok] * codes[tok][ch]
//        (16x16x32 f16 over two chunks, or 16x16x16 for one; eight
//        16-channel tiles)
// Dequantization is folded: logit = s_K * (q'.c) + z_K * sum(q'), and
// o' = sum (p s_V) c + (sum p z_V) on every channel, so codes enter the MFMA
// as small integers.  A code c in bits 2k..2k+1 of a 16-bit half is turned
// into the f16 subnormal c * 2^(2k-24) by a single AND (two codes per dword
// and instruction); the power of two is compensated on the other operand
// (QK) or once at the end (PV).  Precision: q' and w = p s_V are split into
// f16 hi + lo parts (about 22 significant bits); the hi and lo parts occupy
// separate MFMA columns (QK) or rows (PV), so the split costs no extra MFMA.
//
// Lane layout (wave64, lane = 16 * gq + n): for a 16-token chunk the QK
// output gives lane (gq, n) tokens 4gq..4gq+3 of column n, which is exactly
// the PV A-operand layout (row n, tokens 4gq..4gq+3), so the softmax weights
// never leave their lanes.  With GP query heads per KV head (padded to a
// power of two in 2..8), columns are (chunk p, hi/lo t, head g) with
// n = 2GP*p + GP*t + g: one QK tile covers 16 / (2GP) chunks.  The running
// max is updated lazily: a tile is rescaled only when a logit exceeds the
// running max by more than 8 (base-2 units), so p <= 256.
#pragma once

#include <algorithm>
#include <climits>
#include <type_traits>

#include "kvq2_decode_common.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));   // cvt_pkrtz result
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kTau = 8.0f;   // lazy-rescale threshold in base-2 logit units

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, true));
}

// a if sel (all ones) else b, as bit operations: the compiler turns a
// lane-dependent choice between two array elements into an indexed private
// array otherwise.
__device__ __forceinline__ float select_bits(uint32_t sel, float a, float b) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, a) & sel) |
                                       (__builtin_bit_cast(uint32_t, b) & ~sel));
}

__device__ __forceinline__ float f16lo(uint32_t v) { return f16_bits_to_float(v & 0xFFFFu); }
__device__ __forceinline__ float f16hi(uint32_t v) { return f16_bits_to_float(v >> 16); }

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return float_to_f16_bits(lo) | (float_to_f16_bits(hi) << 16);
}

// 16 K codes (channels 0..15 of a 32-bit word) -> two 8-wide f16 operands.
// even: channels (0,8) (1,9) (2,10) (3,11) at scales 2^-24, 2^-22, 2^-20, 2^-18
// odd:  channels (4,12) (5,13) (6,14) (7,15) at scales 2^-16, 2^-22, 2^-20, 2^-18
__device__ __forceinline__ void k_operands(uint32_t w, half8_t& even, half8_t& odd) {
  const uint32_t x = w >> 8;
  const u32x4_t e = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u};
  const u32x4_t o = {w & 0x03000300u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u};
  even = __builtin_bit_cast(half8_t, e);
  odd = __builtin_bit_cast(half8_t, o);
}

// Tile geometry: NPT = chunks_per_tile(GP) chunks per tile.  In LDS a tile
// is stored as [codes of chunk 0..NPT-1 (1024 B each)][scale/zero params
// (128 B each)]; at least 256 B of params space so one 64-lane dword DMA
// always fits.  SHARED: the eight-head layout, whose QK columns are the same
// for both chunks of a tile (every lane takes logits of both chunks).
template <int GP, int NG>
struct Geo {
  static constexpr int NPT = chunks_per_tile(GP);
  static constexpr bool SHARED = 2 * GP * NPT > 16;
  static constexpr int NBLK = 16 / (2 * GP);         // column blocks of the QK tile
  // QK column sets per chunk: each block of a set holds one quantization
  // group's channels; a second set when the blocks are fewer than the groups
  static constexpr int SETS = (!SHARED && NG > NBLK) ? NG / NBLK : 1;
  static constexpr int PARAM_BYTES = NPT >= 2 ? NPT * 128 * NG : 256;
  static constexpr int TILE = NPT * 1024 + PARAM_BYTES;
  static constexpr int RING = NG > 1 ? (NPT >= 4 ? 2 : 3)
                                     : (NPT >= 4 ? 2 : (NPT == 2 ? 4 : 6));   // tiles per wave ring
  static constexpr int PARAM_DMA = NG * ((NPT + 1) / 2);   // 64-lane dword loads of params
  static constexpr int CHUNK_BYTES = 1024 + 128 * NG;
};

// The eight-head kernel keeps its ring in one array, so that the epilogue's
// o' staging (16 KiB) fits in ring positions 0 and 1 and three work-groups
// fit a CU's LDS.
template <int GP, int NG>
__device__ __forceinline__ uint8_t* shared_ring() {
  __shared__ __attribute__((aligned(16))) uint8_t ring[Geo<GP, NG>::RING][4][Geo<GP, NG>::TILE];
  return &ring[0][0][0];
}

// One LDS array per ring position (all waves' slots for that position), so
// that the wait before reading a slot covers only that slot's DMA loads.
template <int GP, int NG, int K>
__device__ __forceinline__ uint8_t* ring_slot(int wave) {
  if constexpr (Geo<GP, NG>::SHARED) {
    return shared_ring<GP, NG>() + (K * 4 + wave) * Geo<GP, NG>::TILE;
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t slot[4][Geo<GP, NG>::TILE];
    return slot[wave];
  }
}

// Per-work-group LDS outside the ring: the waves' softmax (m, l) and, when
// ring position 0 is too small for it, the waves' o' staging.
template <int GP, int NG>
struct WaveStage {
  static constexpr bool kWoInRing =
      (Geo<GP, NG>::SHARED ? Geo<GP, NG>::RING : 1) * 4 * Geo<GP, NG>::TILE >=
      int(4 * GP * kHeadDim * sizeof(float));
  // ring positions holding the token-slice role's q' and softmax weights
  // (clear of the o' staging)
  static constexpr int kQsPos = Geo<GP, NG>::SHARED ? 2 : 1;
  static constexpr int kPbPos = Geo<GP, NG>::SHARED ? 3 : (Geo<GP, NG>::RING >= 3 ? 2 : 1);
  static constexpr int kPbOff = Geo<GP, NG>::SHARED || Geo<GP, NG>::RING >= 3 ? 0 : 4096;
};
template <int GP>
__device__ __forceinline__ float (*wave_m())[GP] {
  __shared__ float m[4][GP];
  return m;
}
template <int GP>
__device__ __forceinline__ float (*wave_l())[GP] {
  __shared__ float l[4][GP];
  return l;
}

template <int GP, int NG>
__device__ __forceinline__ uint8_t* ring_slot_k(int k, int wave) {
  // k is a compile-time constant after unrolling
  if (k == 0) return ring_slot<GP, NG, 0>(wave);
  if (k == 1) return ring_slot<GP, NG, 1>(wave);
  if (k == 2) return ring_slot<GP, NG, 2>(wave);
  if (k == 3) return ring_slot<GP, NG, 3>(wave);
  if (k == 4) return ring_slot<GP, NG, 4>(wave);
  return ring_slot<GP, NG, 5>(wave);
}

template <int GP, int NG>
__device__ __forceinline__ float (*wave_o())[GP][kHeadDim] {
  constexpr bool in_ring = WaveStage<GP, NG>::kWoInRing;
  __shared__ float own[in_ring ? 1 : 4][in_ring ? 1 : GP][kHeadDim];
  return in_ring ? reinterpret_cast<float (*)[GP][kHeadDim]>(ring_slot<GP, NG, 0>(0))
                 : reinterpret_cast<float (*)[GP][kHeadDim]>(&own[0][0][0]);
}

// Direct HBM -> LDS loads and the LDS reads of a tile are written in
// assembly so that the compiler does not serialise them: it cannot tell the
// ring slots apart and would otherwise wait for every outstanding DMA before
// any LDS read.  The kernel waits explicitly (vmcnt) for the one tile it
// reads; no other vector-memory instruction is issued inside the tile loop.
// The outputs of an assembly block of several loads are early-clobber: a
// load's destination must not share a register with an address that a later
// load of the block still reads.
// M0 holds the LDS destination; lane i writes size bytes at M0 + size * i.
// The loads carry the non-temporal hint (NT) when a chunk is read once: on
// the MI355X the scattered 1152-byte chunk pattern streams at ~6.55 TB/s
// with it against ~5.85 TB/s without (global->LDS probe, 2.1 GB of chunks).
// Chunks that several waves read at about the same time (a shared prefix's
// row sets) are loaded without it, so that the L2 serves all but the first.

// 16 bytes per lane from sbase + voff.
template <bool NT = true>
__device__ __forceinline__ void dma_x4(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory", "m0");
}

// 4 bytes per lane from a per-lane address.
template <bool NT = true>
__device__ __forceinline__ void dma_x1(const uint8_t* vaddr, uint32_t lds) {
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off nt"
        :
        : "v"(vaddr), "s"(lds)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off"
        :
        : "v"(vaddr), "s"(lds)
        : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// One piece of (b, h): the INT2 tiles [t_lo, t_hi) of its range of W_b
// virtual tiles (the first piece_cost of them stand for no tile; the rest
// are clipped to the tiles the sequence has, past its first `skip` tiles,
// which a shared-prefix group reads).  Leaves its partial in slot part_slot
// for the combine kernel.
//
// Row-set mode (RS): a piece of a shared-prefix group's item.  The tiles
// are the group's first `skip` tiles of sequence b (any member: they share
// those pages), reached through virtual offsets of rs_cost per tile; every
// wave takes every tile, for the query rows of its own member sequence bq_b,
// and leaves its own partial in slot part_slot + wave.  The four waves
// stream the same tiles at about the same time through their own rings,
// with cache-allocating loads: the first brings a tile into the L2 and the
// others read it there, so memory serves it once for up to four members,
// while the waves stay as independent as in a plain piece.
template <int GP, int NG, bool RS = false>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, const int b, const int h,
                                            const int t_lo, const int t_hi,
                                            const int64_t part_slot, const int skip = 0,
                                            const int bq_b = 0) {
  constexpr int NPT = Geo<GP, NG>::NPT;    // 16-token chunks per tile
  constexpr int RING = Geo<GP, NG>::RING;
  constexpr int TILE = Geo<GP, NG>::TILE;
  float (*wm)[GP] = wave_m<GP>();
  float (*wl)[GP] = wave_l<GP>();
  // Per-wave o' staging of the epilogue; it reuses ring position 0 when that
  // is large enough (the ring is idle by then).
  float (*wo)[GP][kHeadDim] = wave_o<GP, NG>();
  const int G = a.group;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The lane id passes through an empty asm statement so that the per-lane
  // constants derived from it are recomputed per piece rather than hoisted
  // out of the work-group's piece loop (which would keep them live
  // throughout).
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int gq = lane >> 4, n = lane & 15;
  const Int2Range rg = int2_range(a, a.seq_len[b], NPT);

  // ---- per-lane roles --------------------------------------------------
  const int j = n % (2 * GP);        // column within its chunk block
  const int pblk = n / (2 * GP);     // chunk of the tile this column belongs to
  const bool is_hi = j < GP;         // hi column (carries the combined logit)
  const int g_col = j % GP;          // query head of this column
  const bool g_ok = g_col < G;

  // QK operand (q' hi/lo in f16, per-lane layout) and this column's logit
  // scale and group sums of q' (one per column set), all prepared by the
  // rotation pre-pass.
  constexpr int SETS = Geo<GP, NG>::SETS;
  half8_t Bq[4];
  float qscale, qbar_s, qbar2;
  {
    const uint32_t* base = a.bq + (int64_t(RS ? bq_b : b) * a.n_kv_heads + h) * kBqWords;
    const uint4* src = reinterpret_cast<const uint4*>(base + lane * 16);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Bq[kk] = __builtin_bit_cast(half8_t, src[kk]);
    const float4 lq = reinterpret_cast<const float4*>(base + kBqOperandWords)[lane];
    qscale = lq.x;
    qbar_s = lq.y;
    qbar2 = lq.z;
    // Pass the loaded values through empty asm statements: the compiler
    // waits for the loads here, once, instead of inside the tile loop, where
    // its vmcnt wait would also drain the in-flight tile DMA.
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(Bq[kk]));
    asm volatile("" : "+v"(qscale), "+v"(qbar_s), "+v"(qbar2));
  }

  int t_begin, t_end;
  if constexpr (RS) {
    // tile t covers virtual offsets (piece_cost + rs_cost (t - 1), piece_cost + rs_cost t]
    auto tile_at = [&](int v) {
      return min(max((v - a.piece_cost + a.rs_cost - 1) / a.rs_cost, 0), skip);
    };
    t_begin = t_lo <= a.piece_cost ? 0 : tile_at(t_lo);
    t_end = t_hi <= a.piece_cost ? 0 : tile_at(t_hi);
  } else {
    const int tiles_own = (rg.cl - rg.cf) / NPT - skip;
    t_begin = skip + min(max(t_lo - a.piece_cost, 0), tiles_own);
    t_end = skip + min(max(t_hi - a.piece_cost, 0), tiles_own);
  }
  const int n_tiles = t_end - t_begin;
  const int c_begin = rg.cf + NPT * t_begin;   // first chunk of this split
  const float log2_sigma = float(a.log2_sigma_v);

  float4_t cpv[8];
#pragma unroll
  for (int J = 0; J < 8; ++J) cpv[J] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m_h[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) m_h[g] = -INFINITY;
  // Logits are kept as lg' = lg / qscale (lg in base-2 units).  m_eff is the
  // running max minus log2(sigma_v), so p' = 2^(lg - m_eff) = sigma_v 2^(lg - m)
  // and w = p' s_V <= 2^8 fits f16; l, z and o' all carry the same factor.
  // thr = (m + tau) / qscale is the lazy-rescale threshold on lg'.
  // Columns of padding heads (g >= G) keep m_eff = thr = +inf: p' = 0.
  // Lanes whose logits are not used (the lo columns, except in the
  // eight-head layout) keep thr = +inf too, so that the rescale test is a
  // plain compare on every lane.
  const bool thr_lane = g_ok && (Geo<GP, NG>::SHARED || is_hi);
  float m_eff = g_ok ? -INFINITY : INFINITY;
  float thr = thr_lane ? -INFINITY : INFINITY;
  float l_lane = 0.f, z_lane = 0.f;
  float zg_lane[NG];                 // sum of p z_V per quantization group (NG > 1)
#pragma unroll
  for (int k = 0; k < NG; ++k) zg_lane[k] = 0.f;

  const uint8_t* pool = a.pool;
  // Chunk byte offsets (wave-uniform, scalar arithmetic).  Every chunk of a
  // tile in the split's range is fully valid; tiles past the range (prefetch
  // overrun) and invalid page entries read chunk 0 (memory-safe; the former
  // are never computed, the latter are a caller error).
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const_i32* bt_row = (const_i32*)(a.block_table + int64_t(b) * a.bt_stride);
  const int cpp_mask = (1 << a.log2_cpp) - 1;
  constexpr int CB = Geo<GP, NG>::CHUNK_BYTES;
  const int64_t head_off = int64_t(h) * (cpp_mask + 1) * CB;
  // page numbers are int32: a 32-bit bound keeps the check on the scalar unit
  const int32_t num_pages32 = static_cast<int32_t>(min(a.num_pages, int64_t(INT32_MAX)));
  struct Pages { int32_t pg[NPT]; };
  auto fetch_pages = [&](int tile, Pages& P) {
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int lp = (c_begin + tile * NPT + p) >> a.log2_cpp;
      P.pg[p] = (tile < n_tiles && lp < a.bt_stride) ? bt_row[lp] : -1;
    }
  };
  // DMA one tile from HBM into an LDS slot: NPT 64-lane x 16 B loads of the
  // code bytes, then 64-lane dword loads of the params of two chunks each.
  const uint32_t hi_half = 0u - uint32_t(lane >> 5);   // all ones on lanes 32-63
  auto issue_tile = [&](int tile, const Pages& P, uint8_t* slot) {
    int64_t off[NPT];
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int c = c_begin + tile * NPT + p;
      const int32_t page = P.pg[p];
      off[p] = (page >= 0 && page < num_pages32)
                   ? int64_t(page) * a.page_bytes + head_off + int64_t(c & cpp_mask) * CB
                   : int64_t(0);
    }
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(slot));
#pragma unroll
    for (int p = 0; p < NPT; ++p) dma_x4<!RS>(pool + off[p], 16u * lane, lds + 1024u * p);
    // params of chunks 2i (lanes 0-31) and 2i + 1 (lanes 32-63), in parts of
    // 128 bytes: part u of the pair at 1024 NPT + 256 (NG i + u)
#pragma unroll
    for (int i = 0; i < (NPT + 1) / 2; ++i) {
      const int p0 = 2 * i, p1 = NPT > 1 ? 2 * i + 1 : 0;
      // lanes 32-63 read chunk p1's params: one wave-uniform difference from
      // chunk p0's, kept per lane by an AND with the lane's mask
      const uint64_t d = uint64_t(off[p1] - off[p0]);
      const int64_t dl = int64_t(d & (uint64_t(hi_half) | (uint64_t(hi_half) << 32)));
      const uint8_t* pb = pool + off[p0] + kKParamsOff;
#pragma unroll
      for (int u = 0; u < NG; ++u)
        dma_x1<!RS>(pb + (dl + (128 * u + 4 * (lane & 31))),
                    lds + 1024u * NPT + 256u * (NG * i + u));
    }
  };
  constexpr int kDmaPerTile = NPT + Geo<GP, NG>::PARAM_DMA;
  // One tile from its LDS slot: QK on the matrix cores, lazy online softmax
  // on the hi lanes, PV on the matrix cores.  `after_reads` runs once the
  // tile's LDS reads have completed: the slot is refilled there, and the
  // next block-table lookup is issued there, so that no lgkmcnt wait of this
  // tile covers it and its latency overlaps the tile's arithmetic.
  auto compute_tile = [&](const uint8_t* slot, auto&& after_reads) {
    // RING tiles of DMA are outstanding (this one and the RING - 1 after
    // it); this tile's is complete once at most RING - 1 tiles' remain
    wait_vmcnt<(RING - 1) * kDmaPerTile>();
    if constexpr (Geo<GP, NG>::SHARED) {
      // Eight heads: the 16 QK columns (head, hi/lo) serve both chunks of
      // the tile.  After the hi + lo column sums, the hi lanes (n < 8) keep
      // the logits of chunk 0 and the lo lanes (n >= 8) take those of chunk
      // 1 (lane n - 8's sums), so every lane runs the softmax of four tokens
      // of one chunk.  One 16x16x32 PV product per channel tile covers both
      // chunks (k-slots 0-3 chunk 0, 4-7 chunk 1): row n < 8 takes the hi
      // parts of head n's weights, row n + 8 the lo parts.
      uint2 kc0, vc0, kc1, vc1;
      uint4 kp, vp;
      const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(slot));
      const uint32_t acode = lds + 32u * n + 8u * gq;
      const uint32_t aprm = lds + 2048u + (is_hi ? 0u : 128u) + 16u * gq;   // own chunk
      asm volatile(
          "ds_read_b64 %0, %6\n\t"
          "ds_read_b64 %1, %6 offset:512\n\t"
          "ds_read_b64 %2, %6 offset:1024\n\t"
          "ds_read_b64 %3, %6 offset:1536\n\t"
          "ds_read_b128 %4, %7\n\t"
          "ds_read_b128 %5, %7 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc0), "=&v"(vc0), "=&v"(kc1), "=&v"(vc1), "=&v"(kp), "=&v"(vp)
          : "v"(acode), "v"(aprm)
          : "memory");
      after_reads();
      float4_t cq[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint2 kcp = p == 0 ? kc0 : kc1;
        half8_t a0, a1, a2, a3;
        k_operands(kcp.x, a0, a1);
        k_operands(kcp.y, a2, a3);
        float4_t c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bq[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bq[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bq[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, Bq[3], c, 0, 0, 0);
        cq[p] = c;
      }
      // Every lane move below runs with all 64 lanes active and its result
      // is chosen with bit operations (a conditional expression around a
      // lane move can become a branch whose moves read inactive lanes).
      const uint32_t hi_sel = 0u - uint32_t(is_hi);
      float lg[4], zv[4];
      uint32_t svb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d0 = cq[0][r] + dpp_f<0x100 + GP>(cq[0][r]);   // valid on hi lanes
        const float d1 = cq[1][r] + dpp_f<0x100 + GP>(cq[1][r]);
        const float d1m = dpp_f<0x110 + GP>(d1);                   // lo lanes: chunk 1
        const float d = select_bits(hi_sel, d0, d1m);
        const uint32_t kpr = r == 0 ? kp.x : r == 1 ? kp.y : r == 2 ? kp.z : kp.w;
        const uint32_t vpr = r == 0 ? vp.x : r == 1 ? vp.y : r == 2 ? vp.z : vp.w;
        lg[r] = fmaf(f16lo(kpr), d, fmaf(f16hi(kpr), qbar_s, 0.f));
        svb[r] = vpr;
        zv[r] = f16hi(vpr);
      }
      const float tmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
      if (__builtin_amdgcn_ballot_w64(tmax > thr) != 0) {
        const float tm = g_ok ? tmax * qscale : -INFINITY;
        float corr[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float mg = wave_max(g_col == g ? tm : -INFINITY);
          const float mo = m_h[g];
          const float mn = fmaxf(mo, mg);
          corr[g] = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
          m_h[g] = mn;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // head of PV row 4gq + r is (4gq + r) % 8
          const float cr = select_bits(0u - uint32_t(gq & 1), corr[4 + r], corr[r]);
#pragma unroll
          for (int J = 0; J < 8; ++J) cpv[J][r] *= cr;
        }
        float cl = corr[0], ml = m_h[0];
#pragma unroll
        for (int g = 1; g < GP; ++g) {
          const uint32_t sel = 0u - uint32_t(g_col == g);
          cl = select_bits(sel, corr[g], cl);
          ml = select_bits(sel, m_h[g], ml);
        }
        l_lane *= cl;
        z_lane *= cl;
        m_eff = g_ok ? ml - log2_sigma : INFINITY;
        thr = thr_lane ? (ml + kTau) / qscale : INFINITY;
      }
      float w[4], pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(lg[r], qscale, -m_eff));
        l_lane += p;
        z_lane = fmaf(p, zv[r], z_lane);
        pr[r] = p;
        w[r] = fmaf(p, f16lo(svb[r]), 0.f);   // (see the four-head path)
      }
      const fp16x2_t h02 = __builtin_amdgcn_cvt_pkrtz(w[0], w[2]);
      const fp16x2_t h13 = __builtin_amdgcn_cvt_pkrtz(w[1], w[3]);
      const uint32_t hi02 = __builtin_bit_cast(uint32_t, h02), hi13 = __builtin_bit_cast(uint32_t, h13);
      const uint32_t lo02 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_pkrtz(fmaf(pr[0], f16lo(svb[0]), -float(h02[0])),
                                               fmaf(pr[2], f16lo(svb[2]), -float(h02[1]))));
      const uint32_t lo13 = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_pkrtz(fmaf(pr[1], f16lo(svb[1]), -float(h13[0])),
                                               fmaf(pr[3], f16lo(svb[3]), -float(h13[1]))));
      // row n < 8: hi parts of chunk 0 (own) and chunk 1 (lane n + 8);
      // row n + 8: lo parts of chunk 0 (lane n) and chunk 1 (own)
      const uint32_t hi02u = dpp_u<0x100 + GP>(hi02), hi13u = dpp_u<0x100 + GP>(hi13);
      const uint32_t lo02d = dpp_u<0x110 + GP>(lo02), lo13d = dpp_u<0x110 + GP>(lo13);
      auto pick = [&](uint32_t a, uint32_t b) { return (a & hi_sel) | (b & ~hi_sel); };
      const u32x4_t ap = {pick(hi02, lo02d), pick(hi13, lo13d), pick(hi02u, lo02),
                          pick(hi13u, lo13)};
      const half8_t A = __builtin_bit_cast(half8_t, ap);
      const uint32_t e0 = vc0.x, e1 = vc0.y, f0 = vc1.x, f1 = vc1.y;
      const uint32_t e0s = e0 >> 8, e1s = e1 >> 8, f0s = f0 >> 8, f1s = f1 >> 8;
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        const uint32_t mask = 0x00030003u << (2 * (J & 3));
        const uint32_t d = J < 4 ? e0 : e1, ds = J < 4 ? e0s : e1s;
        const uint32_t f = J < 4 ? f0 : f1, fs = J < 4 ? f0s : f1s;
        const u32x4_t bv = {d & mask, ds & mask, f & mask, fs & mask};
        cpv[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bv),
                                                        cpv[J], 0, 0, 0);
      }
      return;
    }
    if constexpr (NG > 1) {
      // ---- quantization groups narrower than the head (NG (s, z) pairs per
      // vector).  Block blk of column set c holds group (c NBLK + blk) mod NG,
      // so the QK product of chunk p gives each block its group's partial
      // dot; every lane scales its block's dot by that group's (s_K, z_K) for
      // every chunk of the tile, the blocks' terms are summed by rotations
      // along the row, and each lane keeps the logits of its own chunk.  PV
      // takes one A operand per group (w = p s_V of that group): a 16-channel
      // output tile lies in one 64-channel group, or (NG = 4) in two
      // 32-channel groups split by output column, taken by two products with
      // the other half of B masked.
      constexpr int NBLK = Geo<GP, NG>::NBLK;
      constexpr int NGB = NG < NBLK ? NG : NBLK;   // distinct groups among a set's blocks
      uint2 kc[NPT], vc[NPT];
      const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(slot));
      const uint32_t acode = lds + 32u * n + 8u * gq;
      if constexpr (NPT == 2) {
        asm volatile(
            "ds_read_b64 %0, %4\n\t"
            "ds_read_b64 %1, %4 offset:512\n\t"
            "ds_read_b64 %2, %4 offset:1024\n\t"
            "ds_read_b64 %3, %4 offset:1536\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kc[0]), "=&v"(vc[0]), "=&v"(kc[1]), "=&v"(vc[1])
            : "v"(acode)
            : "memory");
      } else {
        static_assert(NPT == 4, "tile geometry");
        asm volatile(
            "ds_read_b64 %0, %8\n\t"
            "ds_read_b64 %1, %8 offset:512\n\t"
            "ds_read_b64 %2, %8 offset:1024\n\t"
            "ds_read_b64 %3, %8 offset:1536\n\t"
            "ds_read_b64 %4, %8 offset:2048\n\t"
            "ds_read_b64 %5, %8 offset:2560\n\t"
            "ds_read_b64 %6, %8 offset:3072\n\t"
            "ds_read_b64 %7, %8 offset:3584\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(kc[0]), "=&v"(vc[0]), "=&v"(kc[1]), "=&v"(vc[1]), "=&v"(kc[2]),
              "=&v"(vc[2]), "=&v"(kc[3]), "=&v"(vc[3])
            : "v"(acode)
            : "memory");
      }
      // params: byte o of chunk p's params at 1024 NPT + 256 (NG (p / 2) +
      // o / 128) + 128 (p % 2) + o % 128 (the DMA layout above)
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(slot);
      auto prm = [&](int p, int o) -> uint32_t {
        return sw[(1024 * NPT + 256 * (NG * (p >> 1) + (o >> 7)) + 128 * (p & 1) + (o & 127)) >>
                  2];
      };
      uint32_t kpw[NPT][SETS][4], vpw[NG][4];
#pragma unroll
      for (int p = 0; p < NPT; ++p)
#pragma unroll
        for (int c = 0; c < SETS; ++c) {
          const int grp = (c * NBLK + pblk) % NG;
#pragma unroll
          for (int r = 0; r < 4; ++r) kpw[p][c][r] = prm(p, 4 * ((4 * gq + r) * NG + grp));
        }
#pragma unroll
      for (int k = 0; k < NG; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) vpw[k][r] = prm(pblk, 64 * NG + 4 * ((4 * gq + r) * NG + k));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      after_reads();
      float E[NPT][4];
      // with two sets, lane gq's codes (channels of group gq NG / 4) enter
      // only the product of their group's set
#pragma unroll
      for (int p = 0; p < NPT; ++p) {
#pragma unroll
        for (int r = 0; r < 4; ++r) E[p][r] = 0.f;
#pragma unroll
        for (int c = 0; c < SETS; ++c) {
          const uint32_t keep = SETS == 1 ? ~0u : 0u - uint32_t((gq * NG / 4) / NBLK == c);
          half8_t a0, a1, a2, a3;
          k_operands(kc[p].x & keep, a0, a1);
          k_operands(kc[p].y & keep, a2, a3);
          float4_t cc = {0.f, 0.f, 0.f, 0.f};
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bq[0], cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bq[1], cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bq[2], cc, 0, 0, 0);
          cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, Bq[3], cc, 0, 0, 0);
          const float qb = c == 0 ? qbar_s : qbar2;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = cc[r] + dpp_f<0x100 + GP>(cc[r]);      // hi + lo columns
            E[p][r] = fmaf(f16lo(kpw[p][c][r]), d, fmaf(f16hi(kpw[p][c][r]), qb, E[p][r]));
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (NGB >= 2) E[p][r] += dpp_f<0x120 + 2 * GP>(E[p][r]);   // row_ror
          if constexpr (NGB >= 4) E[p][r] += dpp_f<0x120 + 4 * GP>(E[p][r]);
        }
      }
      float lg[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lg[r] = E[0][r];
#pragma unroll
        for (int p = 1; p < NPT; ++p)
          if (pblk == p) lg[r] = E[p][r];
      }
      float tmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
      if (__builtin_amdgcn_ballot_w64(tmax > thr) != 0) {
        const float tm = (is_hi && g_ok) ? tmax * qscale : -INFINITY;
        float corr[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float mg = wave_max(g_col == g ? tm : -INFINITY);
          const float mo = m_h[g];
          const float mn = fmaxf(mo, mg);
          corr[g] = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
          m_h[g] = mn;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float cr = corr[r % GP];        // head of PV row 4gq + r is (4gq + r) % GP
#pragma unroll
          for (int J = 0; J < 8; ++J) cpv[J][r] *= cr;
        }
        float cl = corr[0], ml = m_h[0];
#pragma unroll
        for (int g = 1; g < GP; ++g) {
          const uint32_t sel = 0u - uint32_t(g_col == g);
          cl = select_bits(sel, corr[g], cl);
          ml = select_bits(sel, m_h[g], ml);
        }
        l_lane *= cl;
#pragma unroll
        for (int k = 0; k < NG; ++k) zg_lane[k] *= cl;
        m_eff = g_ok ? ml - log2_sigma : INFINITY;
        thr = thr_lane ? (ml + kTau) / qscale : INFINITY;
      }
      float w[NG][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(lg[r], qscale, -m_eff));
        l_lane += p;                     // lo lanes accumulate garbage, masked at the end
#pragma unroll
        for (int k = 0; k < NG; ++k) {
          zg_lane[k] = fmaf(p, f16hi(vpw[k][r]), zg_lane[k]);
          w[k][r] = p * f16lo(vpw[k][r]);
        }
      }
      // A operands per group: f16 hi/lo split of w, lo parts moved GP lanes
      // up into the lo rows
      uint32_t av0[NG], av1[NG];
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const fp16x2_t h02 = __builtin_amdgcn_cvt_pkrtz(w[k][0], w[k][2]);
        const fp16x2_t h13 = __builtin_amdgcn_cvt_pkrtz(w[k][1], w[k][3]);
        const uint32_t hi02 = __builtin_bit_cast(uint32_t, h02);
        const uint32_t hi13 = __builtin_bit_cast(uint32_t, h13);
        const uint32_t lo02 = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_pkrtz(w[k][0] - float(h02[0]), w[k][2] - float(h02[1])));
        const uint32_t lo13 = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_pkrtz(w[k][1] - float(h13[0]), w[k][3] - float(h13[1])));
        const uint32_t lo02s = dpp_u<0x110 + GP>(lo02), lo13s = dpp_u<0x110 + GP>(lo13);
        av0[k] = is_hi ? hi02 : lo02s;
        av1[k] = is_hi ? hi13 : lo13s;
      }
      const uint32_t col_lo = 0u - uint32_t(n < 8), col_hi = ~col_lo;
#pragma unroll
      for (int pp = 0; pp < NPT; pp += 2) {
        const uint32_t e0 = vc[pp].x, e1 = vc[pp].y, f0 = vc[pp + 1].x, f1 = vc[pp + 1].y;
        const uint32_t e0s = e0 >> 8, e1s = e1 >> 8, f0s = f0 >> 8, f1s = f1 >> 8;
        auto a_op = [&](int k) {
          const u32x4_t ap = {pblk == pp ? av0[k] : 0u, pblk == pp ? av1[k] : 0u,
                              pblk == pp + 1 ? av0[k] : 0u, pblk == pp + 1 ? av1[k] : 0u};
          return __builtin_bit_cast(half8_t, ap);
        };
#pragma unroll
        for (int J = 0; J < 8; ++J) {
          const uint32_t mask = 0x00030003u << (2 * (J & 3));
          const uint32_t d = J < 4 ? e0 : e1, ds = J < 4 ? e0s : e1s;
          const uint32_t f = J < 4 ? f0 : f1, fs = J < 4 ? f0s : f1s;
          const u32x4_t bv = {d & mask, ds & mask, f & mask, fs & mask};
          if constexpr (NG == 2) {
            cpv[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(J >> 2),
                                                            __builtin_bit_cast(half8_t, bv),
                                                            cpv[J], 0, 0, 0);
          } else {
            // the code mask of this J, restricted to the lane's output column
            // half (lane-constant, so no extra operation per dword)
            const uint32_t ml = mask & col_lo, mh = mask & col_hi;
            const u32x4_t bl = {d & ml, ds & ml, f & ml, fs & ml};
            const u32x4_t bh = {d & mh, ds & mh, f & mh, fs & mh};
            cpv[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(2 * (J >> 2)),
                                                            __builtin_bit_cast(half8_t, bl),
                                                            cpv[J], 0, 0, 0);
            cpv[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_op(2 * (J >> 2) + 1),
                                                            __builtin_bit_cast(half8_t, bh),
                                                            cpv[J], 0, 0, 0);
          }
        }
      }
      return;
    } else {
    uint2 kc[NPT], vc[NPT];
    uint4 kp, vp;
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(slot));
    const uint32_t acode = lds + 32u * n + 8u * gq;
    const uint32_t aprm = lds + 1024u * NPT + 128u * pblk + 16u * gq;
    if constexpr (NPT == 1) {
      asm volatile(
          "ds_read_b64 %0, %4\n\t"
          "ds_read_b64 %1, %4 offset:512\n\t"
          "ds_read_b128 %2, %5\n\t"
          "ds_read_b128 %3, %5 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc[0]), "=&v"(vc[0]), "=&v"(kp), "=&v"(vp)
          : "v"(acode), "v"(aprm)
          : "memory");
    } else if constexpr (NPT == 2) {
      asm volatile(
          "ds_read_b64 %0, %6\n\t"
          "ds_read_b64 %1, %6 offset:512\n\t"
          "ds_read_b64 %2, %6 offset:1024\n\t"
          "ds_read_b64 %3, %6 offset:1536\n\t"
          "ds_read_b128 %4, %7\n\t"
          "ds_read_b128 %5, %7 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc[0]), "=&v"(vc[0]), "=&v"(kc[1]), "=&v"(vc[1]), "=&v"(kp), "=&v"(vp)
          : "v"(acode), "v"(aprm)
          : "memory");
    } else {
      static_assert(NPT == 4, "tile geometry");
      asm volatile(
          "ds_read_b64 %0, %10\n\t"
          "ds_read_b64 %1, %10 offset:512\n\t"
          "ds_read_b64 %2, %10 offset:1024\n\t"
          "ds_read_b64 %3, %10 offset:1536\n\t"
          "ds_read_b64 %4, %10 offset:2048\n\t"
          "ds_read_b64 %5, %10 offset:2560\n\t"
          "ds_read_b64 %6, %10 offset:3072\n\t"
          "ds_read_b64 %7, %10 offset:3584\n\t"
          "ds_read_b128 %8, %11\n\t"
          "ds_read_b128 %9, %11 offset:64\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc[0]), "=&v"(vc[0]), "=&v"(kc[1]), "=&v"(vc[1]), "=&v"(kc[2]), "=&v"(vc[2]),
            "=&v"(kc[3]), "=&v"(vc[3]), "=&v"(kp), "=&v"(vp)
          : "v"(acode), "v"(aprm)
          : "memory");
    }
    after_reads();
    float4_t cq[NPT];
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      half8_t a0, a1, a2, a3;
      k_operands(kc[p].x, a0, a1);
      k_operands(kc[p].y, a2, a3);
      float4_t c = {0.f, 0.f, 0.f, 0.f};
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Bq[0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Bq[1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, Bq[2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a3, Bq[3], c, 0, 0, 0);
      cq[p] = c;
    }
    float4_t c4 = cq[0];
#pragma unroll
    for (int p = 1; p < NPT; ++p)
      if (pblk == p) c4 = cq[p];
    float lg[4], zv[4];
    uint32_t svb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float d = c4[r] + dpp_f<0x100 + GP>(c4[r]);          // hi + lo columns
      const uint32_t kpr = r == 0 ? kp.x : r == 1 ? kp.y : r == 2 ? kp.z : kp.w;
      const uint32_t vpr = r == 0 ? vp.x : r == 1 ? vp.y : r == 2 ? vp.z : vp.w;
      lg[r] = fmaf(f16lo(kpr), d, fmaf(f16hi(kpr), qbar_s, 0.f));          // lg' = s_K d + z_K sum(q')/qscale
      svb[r] = vpr;
      zv[r] = f16hi(vpr);
    }
    // lazy running max
    float tmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__builtin_amdgcn_ballot_w64(tmax > thr) != 0) {
      const float tm = (is_hi && g_ok) ? tmax * qscale : -INFINITY;
      float corr[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float mg = wave_max(g_col == g ? tm : -INFINITY);
        const float mo = m_h[g];
        const float mn = fmaxf(mo, mg);
        corr[g] = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
        m_h[g] = mn;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // head of PV row 4gq + r is (4gq + r) % GP
        float cr = corr[r % GP];
        if constexpr (GP == 8) cr = select_bits(0u - uint32_t(gq & 1), corr[4 + r], corr[r]);
#pragma unroll
        for (int J = 0; J < 8; ++J) cpv[J][r] *= cr;
      }
      float cl = corr[0], ml = m_h[0];
#pragma unroll
      for (int g = 1; g < GP; ++g) {
        const uint32_t sel = 0u - uint32_t(g_col == g);
        cl = select_bits(sel, corr[g], cl);
        ml = select_bits(sel, m_h[g], ml);
      }
      l_lane *= cl;
      z_lane *= cl;
      m_eff = g_ok ? ml - log2_sigma : INFINITY;
      thr = thr_lane ? (ml + kTau) / qscale : INFINITY;
    }
    // Products with an f16 operand are written as fmaf(x, f16, 0): each is
    // then one mixed-precision FMA instead of a conversion and a multiply
    // (the same value: one rounding of the exact product; the kernel is
    // bound by VALU issue as much as by HBM, so every instruction per tile
    // counts).
    float w[4], pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(lg[r], qscale, -m_eff));
      l_lane += p;                       // lo lanes accumulate garbage, masked at the end
      z_lane = fmaf(p, zv[r], z_lane);
      pr[r] = p;
      w[r] = fmaf(p, f16lo(svb[r]), 0.f);
    }
    // f16 hi/lo split of w (each part packed two per dword, rounded toward
    // zero: lo = p s_V - hi, one FMA, carries the remainder, so hi + lo is w
    // to ~2^-20); lo parts move GP lanes up (row_shr) into the lo rows
    const fp16x2_t h02 = __builtin_amdgcn_cvt_pkrtz(w[0], w[2]);
    const fp16x2_t h13 = __builtin_amdgcn_cvt_pkrtz(w[1], w[3]);
    const uint32_t hi02 = __builtin_bit_cast(uint32_t, h02), hi13 = __builtin_bit_cast(uint32_t, h13);
    const uint32_t lo02 = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_pkrtz(fmaf(pr[0], f16lo(svb[0]), -float(h02[0])),
                                             fmaf(pr[2], f16lo(svb[2]), -float(h02[1]))));
    const uint32_t lo13 = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_pkrtz(fmaf(pr[1], f16lo(svb[1]), -float(h13[0])),
                                             fmaf(pr[3], f16lo(svb[3]), -float(h13[1]))));
    const uint32_t lo02s = dpp_u<0x110 + GP>(lo02), lo13s = dpp_u<0x110 + GP>(lo13);
    const uint32_t av0 = is_hi ? hi02 : lo02s;
    const uint32_t av1 = is_hi ? hi13 : lo13s;
    if constexpr (NPT >= 2) {
      // Two chunks per 16x16x32 product: k-slots 0-3 hold tokens 4gq..4gq+3
      // of chunk pp, slots 4-7 the same tokens of chunk pp + 1; a row (a
      // column of the QK tile) carries weights only in the half of its own
      // chunk, so each row still accumulates its own chunk's tokens.
#pragma unroll
      for (int pp = 0; pp < NPT; pp += 2) {
        const u32x4_t ap = {pblk == pp ? av0 : 0u, pblk == pp ? av1 : 0u,
                            pblk == pp + 1 ? av0 : 0u, pblk == pp + 1 ? av1 : 0u};
        const half8_t A = __builtin_bit_cast(half8_t, ap);
        const uint32_t e0 = vc[pp].x, e1 = vc[pp].y, f0 = vc[pp + 1].x, f1 = vc[pp + 1].y;
        const uint32_t e0s = e0 >> 8, e1s = e1 >> 8, f0s = f0 >> 8, f1s = f1 >> 8;
#pragma unroll
        for (int J = 0; J < 8; ++J) {
          const uint32_t mask = 0x00030003u << (2 * (J & 3));
          const uint32_t d = J < 4 ? e0 : e1, ds = J < 4 ? e0s : e1s;
          const uint32_t f = J < 4 ? f0 : f1, fs = J < 4 ? f0s : f1s;
          const u32x4_t bv = {d & mask, ds & mask, f & mask, fs & mask};
          cpv[J] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bv),
                                                          cpv[J], 0, 0, 0);
        }
      }
    } else {
      const u32x2_t ap = {av0, av1};
      const half4_t A = __builtin_bit_cast(half4_t, ap);
      const uint32_t d0 = vc[0].x, d1 = vc[0].y;
      const uint32_t d0s = d0 >> 8, d1s = d1 >> 8;
#pragma unroll
      for (int J = 0; J < 8; ++J) {
        const uint32_t mask = 0x00030003u << (2 * (J & 3));
        const uint32_t d = J < 4 ? d0 : d1, ds = J < 4 ? d0s : d1s;
        const u32x2_t bv = {d & mask, ds & mask};
        cpv[J] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(half4_t, bv), cpv[J],
                                                       0, 0, 0);
      }
    }
    }   // NG == 1
  };

  // ---- tile loop: a ring of RING LDS tile slots per wave.  A slot is
  // refilled with the tile RING steps ahead as soon as its LDS reads have
  // completed (inside compute_tile), so RING tiles are in flight while one
  // is computed.  Every computed step issues its DMA unconditionally (tiles
  // past the end read chunk 0 and are never computed), so the number of
  // loads in flight at each wait is the same on every path; page lookups
  // run one step ahead of the DMA.
  // tiles wave, wave + 4, ... (row-set mode: every tile)
  constexpr int kStep = RS ? 1 : 4;
  const int first = RS ? 0 : wave;
  const int my_tiles = RS ? n_tiles : (n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0);
  if (my_tiles > 0) {
    Pages pn;
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      fetch_pages(first + kStep * k, pn);
      issue_tile(first + kStep * k, pn, ring_slot_k<GP, NG>(k, wave));
    }
    fetch_pages(first + kStep * RING, pn);
    for (int k0 = 0; k0 < my_tiles; k0 += RING) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        if (k0 + k < my_tiles) {
          const int ahead = first + kStep * (k0 + k + RING);
          uint8_t* slot = ring_slot_k<GP, NG>(k, wave);
          // Rotating wave priority: the arbiter otherwise serves the oldest
          // resident waves first, and the work-groups of one CU, which all
          // carry equal work, would finish far apart.  With a ring of a
          // multiple of four slots the priority is the slot's position, a
          // constant of the unrolled loop (one instruction per tile, no
          // branches; measured 1-4 us faster per call than a phase that also
          // depends on the work-group), else it also turns with the
          // work-group index.
          const int pr = RING % 4 == 0 ? k & 3 : (k0 + k + int(blockIdx.x)) & 3;
          if (pr == 0) __builtin_amdgcn_s_setprio(0);
          else if (pr == 1) __builtin_amdgcn_s_setprio(1);
          else if (pr == 2) __builtin_amdgcn_s_setprio(2);
          else __builtin_amdgcn_s_setprio(3);
          compute_tile(slot, [&] {
            issue_tile(ahead, pn, slot);
            fetch_pages(ahead + kStep, pn);
          });
        }
      }
    }
    wait_vmcnt<0>();     // drain DMA before the ring memory is reused
  }
  // The epilogue and the partial store are short and end the piece: they
  // run at the top priority so that streaming waves of other work-groups do
  // not starve them.
  __builtin_amdgcn_s_setprio(3);
  __syncthreads();   // the ring is idle from here on

  // ---- wave epilogue: per-head l, z and o' into LDS -----------------------
  float l_h[GP], z_h[GP];
  // (in the eight-head layout the lo lanes hold the sums of the tiles'
  // second chunks, for the same heads)
  constexpr bool kAllLanes = Geo<GP, NG>::SHARED;
  // (with NG groups: the zero term of each group, per head)
  float zk_h[GP][NG];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    l_h[g] = wave_sum(((kAllLanes || is_hi) && g_col == g) ? l_lane : 0.f);
    if constexpr (NG == 1) {
      z_h[g] = wave_sum(((kAllLanes || is_hi) && g_col == g) ? z_lane : 0.f);
    } else {
      z_h[g] = 0.f;
#pragma unroll
      for (int k = 0; k < NG; ++k) zk_h[g][k] = wave_sum((is_hi && g_col == g) ? zg_lane[k] : 0.f);
    }
  }
#pragma unroll
  for (int J = 0; J < 8; ++J) {
    const float sc = ldexpf(1.0f, 24 - 2 * (J & 3));
    const int ch = 64 * (J >> 2) + 4 * n + (J & 3);
    if constexpr (GP <= 4) {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        float v = 0.f;
#pragma unroll
        for (int r = g; r < 4; r += GP) v += cpv[J][r];
        v = xor32_sum(xor16_sum(v));
        float zz = z_h[g];
        if constexpr (NG == 2) zz = zk_h[g][J >> 2];
        if constexpr (NG == 4)
          zz = select_bits(0u - uint32_t(n < 8), zk_h[g][2 * (J >> 2)], zk_h[g][2 * (J >> 2) + 1]);
        if (gq == 0 && g < G) wo[wave][g][ch] = v * sc + zz;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = xor32_sum(cpv[J][r]);
        const int g = 4 * (gq & 1) + r;
        const float zg = select_bits(0u - uint32_t(gq & 1), z_h[4 + r], z_h[r]);
        if (gq < 2 && g < G) wo[wave][g][ch] = v * sc + zg;
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
      if (g < G) { wm[wave][g] = m_h[g] - log2_sigma; wl[wave][g] = l_h[g]; }
  }

  __syncthreads();
  if constexpr (RS) store_wave_partials<GP>(G, wm, wl, wo, a.partials + part_slot * G * kPartialStride);
  else store_partial<GP>(G, wm, wl, wo, a.partials + part_slot * G * kPartialStride);
}

// Decode over equal tile ranges: the virtual tiles of all (b, h), in order,
// W_b = max(1, INT2 tiles of sequence b) + piece_cost per (b, h), are cut
// into gridDim.x equal contiguous ranges, one per work-group (one round of
// resident work-groups, so no work queue and no tail of late items).  A
// work-group takes every (b, h) its range touches.  Partial slot of
// (work-group i, pair p) is i + p: the (i, p) overlaps form a monotone path,
// so the slots are unique and those of one pair are contiguous.
// Token-by-token list of (b, h), slice z: tokens [64 z, 64 z + 64) of the
// list (the bf16 sink, the INT2 positions outside whole tiles, the bf16
// recent window), one 16-token tile per wave, plain fp32, merged into one
// partial in slot tok_slot0 + (b Hkv + h) n_tok_slices + z for the combine.
// Run by the work-groups after the streaming ones: they are dispatched as
// the streaming work-groups retire, into the CUs that the end of the stream
// leaves idle.  q' comes from the pre-pass; the LDS buffers are carved from
// the (idle) ring.
template <int GP, int NG>
__device__ void token_slice_item(const DecodeArgs& a, int idx) {
  constexpr int NPT = Geo<GP, NG>::NPT;
  __shared__ float qsum[GP];
  __shared__ int qexp[GP];
  const int S = a.n_tok_slices;
  const int z = idx % S, pair = idx / S;
  const int b = pair / a.n_kv_heads, h = pair % a.n_kv_heads;
  const int G = a.group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float (*qs)[kHeadDim] =
      reinterpret_cast<float (*)[kHeadDim]>(ring_slot<GP, NG, WaveStage<GP, NG>::kQsPos>(0));
  float (*pbuf)[16][GP] = reinterpret_cast<float (*)[16][GP]>(
      ring_slot<GP, NG, WaveStage<GP, NG>::kPbPos>(0) + WaveStage<GP, NG>::kPbOff);
  float (*wm)[GP] = wave_m<GP>();
  float (*wl)[GP] = wave_l<GP>();
  float (*wo)[GP][kHeadDim] = wave_o<GP, NG>();
  load_queries<GP>(a, b, h, qs, qsum, qexp);
  // with NG quantization groups, sum(q') over each 32-channel quarter
  __shared__ float qsum4[GP][4];
  if constexpr (NG > 1) {
    if (tid < G * 4) {
      const int g = tid >> 2, k = tid & 3;
      float sum = 0.f;
      for (int c = 0; c < 32; ++c) sum += qs[g][32 * k + c];
      qsum4[g][k] = sum;
    }
    __syncthreads();
  }
  const int L = a.seq_len[b];
  const Int2Range rg = int2_range(a, L, NPT);
  const TokenList tl = token_list(a, L, rg);
  float m[GP], l[GP], acc0[GP], acc1[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) { m[g] = -INFINITY; l[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }
  token_tile<GP>(a, b, h, tl, rg, 4 * z + wave, qs, qsum, qsum4, pbuf[wave], m, l, acc0,
             acc1);
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < G) {
      wo[wave][g][2 * lane] = acc0[g];
      wo[wave][g][2 * lane + 1] = acc1[g];
      if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
    }
  }
  __syncthreads();
  float* stage = &wo[0][0][0];
  merge_wave_states<GP>(G, wm, wl, wo, stage);
  float* out = a.partials + (a.tok_slot0 + int64_t(pair) * S + z) * G * kPartialStride;
  for (int i = tid; i < G * kPartialStride; i += blockDim.x) out[i] = stage[i];
}

// A row-set piece of a shared-prefix group: group gidx, KV head h, row set
// r (members 4r .. 4r + 3 of the group, one per wave; a wave without a valid
// member takes the representative's rows and its partial is not read).
template <int GP, int NG>
__device__ __forceinline__ void rowset_piece(const DecodeArgs& a, int gidx, int h, int r,
                                             int64_t q, int i, int t_lo, int t_hi) {
  const int32_t* gi = a.grp_info + int64_t(gidx) * kGrpInfo;
  const int skip = gi[kGiSkip], rep = gi[kGiRep];
  const int m = gi[kGiMemberStart] + 4 * r + (threadIdx.x >> 6);
  int bw = rep;
  if (m < gi[kGiMemberEnd]) {
    const int bb = a.members[m];
    if (bb >= 0 && bb < a.batch && a.seq_group[bb] == gidx && a.seq_member[bb] == m) bw = bb;
  }
  decode_item<GP, NG, true>(a, rep, h, t_lo, t_hi, a.rs_slot0 + (int64_t(i) + q) * 4, skip,
                            __builtin_amdgcn_readfirstlane(bw));
}

// PRE: the decode has shared-prefix groups (one (scale, zero) pair per
// vector); their row-set items follow the (b, h) pieces.
template <int GP, int NG, bool PRE = false>
__global__ __launch_bounds__(256, GP <= 4 ? (NG == 1 ? 4 : 3) : 2) void decode_mfma_kernel(
    DecodeArgs a) {
  if (static_cast<int>(blockIdx.x) >= a.chain_groups) {
    token_slice_item<GP, NG>(a, static_cast<int>(blockIdx.x) - a.chain_groups);
    return;
  }
  // (low 32 bits of the 100 MHz clock: differences wrap correctly; held in
  // a vector register, the scalar ones being the scarcer here)
  uint32_t t_start = static_cast<uint32_t>(__builtin_amdgcn_s_memrealtime());
  asm volatile("" : "+v"(t_start));
  const int i = blockIdx.x;
  const int Hkv = a.n_kv_heads, B = a.batch;
  const int32_t* pre = a.tile_prefix;
  const int g0 = a.range_start[i], g1 = a.range_start[i + 1];
  if (g0 >= g1) return;
  // virtual tiles of the (b, h) pieces; a shared-prefix decode's row-set
  // items follow them
  const int pairs_total = PRE ? Hkv * pre[B] : INT_MAX;
  bool first = true;
  if (g0 < pairs_total) {
    // sequence holding tile g0: the largest b with Hkv * pre[b] <= g0
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (Hkv * pre[mid] <= g0) lo = mid; else hi = mid;
    }
    int b = lo;
    int wb = pre[b + 1] - pre[b];
    int h = (g0 - Hkv * pre[b]) / wb;
    for (;;) {
      const int sp = Hkv * pre[b] + h * wb;   // first tile of (b, h)
      if (sp >= g1) break;
      if (!first) __syncthreads();   // the previous piece is done with every LDS buffer
      first = false;
      const int p = b * Hkv + h;
      const int skip = PRE ? a.seq_skip[b] : 0;
      decode_item<GP, NG>(a, __builtin_amdgcn_readfirstlane(b), __builtin_amdgcn_readfirstlane(h),
                          max(g0, sp) - sp, min(g1, sp + wb) - sp, int64_t(i) + p,
                          __builtin_amdgcn_readfirstlane(skip));
      if (++h == Hkv) {
        h = 0;
        if (++b == B) break;
        wb = pre[b + 1] - pre[b];
      }
    }
  }
  if (PRE && g1 > pairs_total) {
    // row-set items: group by group, (h, r) in order within a group
    const int v0 = max(g0, pairs_total) - pairs_total, v1 = g1 - pairs_total;
    const int32_t* gi = a.grp_info;
    // the largest group whose items start at or before v0 (groups without
    // items share their successor's start and are passed over)
    int lo = 0, hi = a.n_groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (gi[int64_t(mid) * kGrpInfo + kGiRsPrefix] <= v0) lo = mid; else hi = mid;
    }
    int gidx = lo;
    int w = gi[int64_t(gidx) * kGrpInfo + kGiWidth];
    int rows = gi[int64_t(gidx) * kGrpInfo + kGiRowSets];
    int start = gi[int64_t(gidx) * kGrpInfo + kGiRsPrefix];
    int idx = rows > 0 ? (v0 - start) / w : 0;
    for (;;) {
      if (idx >= Hkv * rows) {   // next group with items
        if (++gidx >= a.n_groups) break;
        w = gi[int64_t(gidx) * kGrpInfo + kGiWidth];
        rows = gi[int64_t(gidx) * kGrpInfo + kGiRowSets];
        start = gi[int64_t(gidx) * kGrpInfo + kGiRsPrefix];
        idx = 0;
        continue;
      }
      const int sq = start + idx * w;   // first virtual tile of the item
      if (sq >= v1) break;
      if (!first) __syncthreads();
      first = false;
      const int64_t q = gi[int64_t(gidx) * kGrpInfo + kGiItemBase] + idx;
      if constexpr (PRE)
        rowset_piece<GP, NG>(a, __builtin_amdgcn_readfirstlane(gidx), idx / rows, idx % rows, q,
                             i, max(v0, sq) - sq, min(v1, sq + w) - sq);
      ++idx;
    }
  }
  // this range's duration, into the cell (dispatch round, XCD) of its index
  // for the next call's weights (vector atomics; one lane)
  if (a.feedback != nullptr && threadIdx.x == 0) {
    const uint32_t dur = static_cast<uint32_t>(__builtin_amdgcn_s_memrealtime()) - t_start;
    const int cell = 8 * min(i / a.round_size, 3) + (i & 7);
    atomicAdd(a.feedback + kFbSum + cell, dur);
    atomicAdd(a.feedback + kFbCnt + cell, 1u);
  }
}

// Split-K combine of (b, h): the pieces' partials (slots i0 + p .. i1 + p,
// p = b Hkv + h, with i0, i1 the first and last range touching it) and its
// token-list slices.  A kernel of its own: it starts once every partial is
// written, with HBM idle, so its few dependent loads are short.  One
// 256-thread work-group per (KV head, sequence) for large batches
// (combine_kernel); one 1024-thread work-group per (KV head, sequence, query
// head) when there are few (sequence, KV head) pairs, so that a small
// batch's combine spreads over more CUs and takes its many splits in one
// round (combine_head_kernel).
// Threads of a combine_kernel work-group: 512 for eight heads (four outputs
// per thread of 256 would hold 250 VGPRs), else 256.  The eight-head
// combine keeps two work-groups per CU (four waves per SIMD, at most 128
// VGPRs), so that the 512 (sequence, KV head) pairs of a 64-sequence batch
// run in one round.
template <int GP>
constexpr int combine_threads() { return GP == 8 ? 512 : 256; }

template <int GP, bool PRE = false>
__global__ __launch_bounds__(combine_threads<GP>(), GP == 8 ? 4 : 1) void combine_kernel(
    DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int p = b * a.n_kv_heads + h;
  const int pr = a.pair_range[p];
  const int i0 = pr & 0xFFFF, i1 = pr >> 16;
  const int64_t tok = a.tok_slot0 + int64_t(p) * a.n_tok_slices;
  int64_t rs = 0;
  const int n_rs = PRE ? rowset_slots(a, b, h, rs) : 0;
  combine_pair<GP, PRE, combine_threads<GP>()>(a, b, h, int64_t(i0) + p, i1 - i0 + 1, tok,
                                              a.n_tok_slices, rs, n_rs);
}

constexpr int kHeadCombineParts = 8;   // 128-thread parts of a combine_head_kernel work-group

template <int GP, bool PRE = false>
__global__ __launch_bounds__(128 * kHeadCombineParts) void combine_head_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int p = b * a.n_kv_heads + h;
  const int pr = a.pair_range[p];
  const int i0 = pr & 0xFFFF, i1 = pr >> 16;
  const int64_t tok = a.tok_slot0 + int64_t(p) * a.n_tok_slices;
  int64_t rs = 0;
  const int n_rs = PRE ? rowset_slots(a, b, h, rs) : 0;
  combine_head<GP, kHeadCombineParts, PRE>(a, b, h, blockIdx.z, int64_t(i0) + p, i1 - i0 + 1,
                                           tok, a.n_tok_slices, rs, n_rs);
}

}  // namespace
}  // namespace kvq
