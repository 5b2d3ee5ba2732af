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
//        (16x16x16 f16, eight 16-channel tiles)
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
// power of two <= 8), columns are (chunk p, hi/lo t, head g) with
// n = 2GP*p + GP*t + g: one QK tile covers 16 / (2GP) chunks.  The running
// max is updated lazily: a tile is rescaled only when a logit exceeds the
// running max by more than 8 (base-2 units), so p <= 256.
#include <type_traits>

#include "kvq2_decode_common.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
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

// Channel and scale exponent of k-slot i (pair q = i/2, element e = i%2) of
// QK k-step kk for lane group gq: channel = 32gq + 16(kk/2) + local, value
// scale 2^(2s - 24).
__device__ __forceinline__ void kslot_channel(int gq, int kk, int i, int& ch, int& s) {
  const int q = i >> 1, e = i & 1;
  const int local = (kk & 1) ? (4 + q + 8 * e) : (q + 8 * e);
  ch = 32 * gq + 16 * (kk >> 1) + local;
  s = (kk & 1) ? (q == 0 ? 4 : q) : q;
}

template <int GP>
struct Tile {
  static constexpr int NPT = 16 / (2 * GP);
  uint2 kc[NPT];
  uint2 vc[NPT];
  uint4 kp;       // K (scale, zero) of tokens 4gq..4gq+3 of this lane's chunk
  uint4 vp;       // V (scale, zero)
  int64_t off[NPT];   // chunk byte offsets; -1 = masked chunk (loads read chunk 0)
};

template <int GP>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NPT = Tile<GP>::NPT;   // 16-token chunks per tile
  __shared__ float qraw[GP][kHeadDim];
  __shared__ float qs[GP][kHeadDim];
  __shared__ float qsum[GP];
  __shared__ float pbuf[4][16][GP];
  __shared__ float wm[4][GP], wl[4][GP];
  __shared__ float wo[4][GP][kHeadDim];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4, n = lane & 15;
  const int L = a.seq_len[b];

  rotate_queries<GP>(a, b, h, qraw, qs, qsum);

  const Int2Range rg = int2_range(a, L, NPT);
  if (s == a.n_split_int2) {
    float m[GP], l[GP], acc0[GP], acc1[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) { m[g] = -INFINITY; l[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }
    token_path<GP>(a, b, h, L, rg, qs, qsum, pbuf, m, l, acc0, acc1);
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      if (g < G) {
        wo[wave][g][2 * lane] = acc0[g];
        wo[wave][g][2 * lane + 1] = acc1[g];
        if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
      }
    }
    __syncthreads();
    finish_work_group<GP>(a, b, h, s, wm, wl, wo, qraw);
    return;
  }

  // ---- per-lane roles --------------------------------------------------
  const int j = n % (2 * GP);        // column within its chunk block
  const int pblk = n / (2 * GP);     // chunk of the tile this column belongs to
  const bool is_hi = j < GP;         // hi column (carries the combined logit)
  const int g_col = j % GP;          // query head of this column
  const bool g_ok = g_col < G;

  // Per-head normalisation 2^-e of q' (max |q'| <= 1 after scaling).
  float qscale, qbar;
  half8_t Bq[4];
  {
    float mx = 0.f;
    if (g_ok) {
      for (int c = 0; c < kHeadDim; ++c) mx = fmaxf(mx, fabsf(qs[g_col][c]));
    }
    const int e = mx > 0.f ? ilogbf(mx) + 1 : 0;
    const float down = ldexpf(1.0f, -e);
    qscale = ldexpf(1.0f, 16 + e);
    qbar = g_ok ? qsum[g_col] : 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int ch, sc;
        kslot_channel(gq, kk, i, ch, sc);
        const float v = g_ok ? qs[g_col][ch] * down * ldexpf(1.0f, 8 - 2 * sc) : 0.f;
        const _Float16 hi = static_cast<_Float16>(v);
        const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
        Bq[kk][i] = is_hi ? hi : lo;
      }
    }
  }

  int t_begin, t_end;
  split_tiles(a, rg, NPT, s, t_begin, t_end);
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
  float m_eff = g_ok ? -INFINITY : INFINITY;
  float thr = g_ok ? -INFINITY : INFINITY;
  float l_lane = 0.f, z_lane = 0.f;
  const float qbar_s = qbar / qscale;

  const uint8_t* pool = a.pool;
  // Chunk byte offsets of a tile (wave-uniform, scalar arithmetic).  Every
  // chunk of a tile in the split's range is fully valid; tiles past the range
  // (prefetch overrun) and invalid page entries read chunk 0 (memory-safe;
  // the former are never computed, the latter are a caller error).
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const_i32* bt_row = (const_i32*)(a.block_table + int64_t(b) * a.bt_stride);
  const int cpp_mask = (1 << a.log2_cpp) - 1;
  const int64_t head_off = int64_t(h) * (cpp_mask + 1) * kChunkBytes;
  // Page numbers of a tile's chunks (-1 outside the split or the table).
  struct Pages { int32_t pg[NPT]; };
  auto fetch_pages = [&](int tile, Pages& P) {
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int lp = (c_begin + tile * NPT + p) >> a.log2_cpp;
      P.pg[p] = (tile < n_tiles && lp < a.bt_stride) ? bt_row[lp] : -1;
    }
  };
  auto tile_offsets = [&](int tile, const Pages& P, Tile<GP>& t) {
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int c = c_begin + tile * NPT + p;
      const int32_t page = P.pg[p];
      t.off[p] = (page >= 0 && page < a.num_pages)
                     ? int64_t(page) * a.page_bytes + head_off + int64_t(c & cpp_mask) * kChunkBytes
                     : int64_t(0);
    }
  };
  auto load_tile = [&](Tile<GP>& t) {
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const uint8_t* ch = pool + t.off[p];
      t.kc[p] = *reinterpret_cast<const uint2*>(ch + kKCodesOff + 32 * n + 8 * gq);
      t.vc[p] = *reinterpret_cast<const uint2*>(ch + kVCodesOff + 32 * n + 8 * gq);
    }
    int64_t mine = t.off[0];
#pragma unroll
    for (int p = 1; p < NPT; ++p) mine = (pblk == p) ? t.off[p] : mine;
    const uint8_t* ch = pool + mine;
    t.kp = *reinterpret_cast<const uint4*>(ch + kKParamsOff + 16 * gq);
    t.vp = *reinterpret_cast<const uint4*>(ch + kVParamsOff + 16 * gq);
  };

  // One tile: QK on the matrix cores, lazy online softmax on the hi lanes,
  // PV on the matrix cores.
  auto compute_tile = [&](const Tile<GP>& t) {
    float4_t cq[NPT];
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      half8_t a0, a1, a2, a3;
      k_operands(t.kc[p].x, a0, a1);
      k_operands(t.kc[p].y, a2, a3);
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
      const uint32_t kpr = r == 0 ? t.kp.x : r == 1 ? t.kp.y : r == 2 ? t.kp.z : t.kp.w;
      const uint32_t vpr = r == 0 ? t.vp.x : r == 1 ? t.vp.y : r == 2 ? t.vp.z : t.vp.w;
      lg[r] = fmaf(f16lo(kpr), d, f16hi(kpr) * qbar_s);          // lg' = s_K d + z_K sum(q')/qscale
      svb[r] = vpr;
      zv[r] = f16hi(vpr);
    }
    // lazy running max
    float tmax = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    if (__any(is_hi && g_ok && tmax > thr)) {
      const float tm = (is_hi && g_ok) ? tmax * qscale : -INFINITY;
      float corr[GP], m_new[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float mg = wave_max(g_col == g ? tm : -INFINITY);
        const float mo = m_h[g];
        m_new[g] = fmaxf(mo, mg);
        corr[g] = (m_new[g] == -INFINITY) ? 1.f : exp2f(mo - m_new[g]);
        m_h[g] = m_new[g];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // head of PV row 4gq + r is (4gq + r) % GP
        float cr = corr[r % GP];
        if constexpr (GP == 8) cr = (gq & 1) ? corr[4 + r] : corr[r];
#pragma unroll
        for (int J = 0; J < 8; ++J) cpv[J][r] *= cr;
      }
      float cl = corr[0], ml = m_h[0];
#pragma unroll
      for (int g = 1; g < GP; ++g) {
        cl = (g_col == g) ? corr[g] : cl;
        ml = (g_col == g) ? m_h[g] : ml;
      }
      l_lane *= cl;
      z_lane *= cl;
      m_eff = g_ok ? ml - log2_sigma : INFINITY;
      thr = g_ok ? (ml + kTau) / qscale : INFINITY;
    }
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(lg[r], qscale, -m_eff));
      l_lane += p;                       // lo lanes accumulate garbage, masked at the end
      z_lane = fmaf(p, zv[r], z_lane);
      w[r] = p * f16lo(svb[r]);
    }
    // f16 hi/lo split of w; lo parts move GP lanes up (row_shr) into the lo rows
    const _Float16 h0 = static_cast<_Float16>(w[0]), h1 = static_cast<_Float16>(w[1]);
    const _Float16 h2 = static_cast<_Float16>(w[2]), h3 = static_cast<_Float16>(w[3]);
    const uint32_t hi02 = pack_f16(float(h0), float(h2)), hi13 = pack_f16(float(h1), float(h3));
    const uint32_t lo02 = pack_f16(w[0] - float(h0), w[2] - float(h2));
    const uint32_t lo13 = pack_f16(w[1] - float(h1), w[3] - float(h3));
    const uint32_t lo02s = dpp_u<0x110 + GP>(lo02), lo13s = dpp_u<0x110 + GP>(lo13);
    const uint32_t av0 = is_hi ? hi02 : lo02s;
    const uint32_t av1 = is_hi ? hi13 : lo13s;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const u32x2_t ap = {pblk == p ? av0 : 0u, pblk == p ? av1 : 0u};
      const half4_t A = __builtin_bit_cast(half4_t, ap);
      const uint32_t d0 = t.vc[p].x, d1 = t.vc[p].y;
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
  };

  // ---- tile loop: a ring of kRing tile buffers, loads kRing-1 tiles ahead --
  // Every step issues its prefetch unconditionally (tiles past the end read
  // chunk 0 and are never computed), so the number of loads in flight is the
  // same on every path and each tile waits only for its own loads.
  constexpr int kRing = 3;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;     // tiles wave, wave+4, ...
  if (my_tiles > 0) {
    // Page lookups run one step ahead of the loads that need them, and the
    // loads kRing-1 tiles ahead of the tile being computed.
    Tile<GP> buf[kRing];
    Pages pn;
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) {
      fetch_pages(wave + 4 * k, pn);
      tile_offsets(wave + 4 * k, pn, buf[k]);
      load_tile(buf[k]);
    }
    fetch_pages(wave + 4 * (kRing - 1), pn);
    for (int k0 = 0; k0 < my_tiles; k0 += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        const int kn = (k + kRing - 1) % kRing;
        const int ahead = wave + 4 * (k0 + k + kRing - 1);
        tile_offsets(ahead, pn, buf[kn]);
        load_tile(buf[kn]);
        fetch_pages(ahead + 4, pn);
        if (k0 + k < my_tiles) compute_tile(buf[k]);
      }
    }
  }

  // ---- wave epilogue: per-head l, z and o' into LDS -----------------------
  float l_h[GP], z_h[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    l_h[g] = wave_sum((is_hi && g_col == g) ? l_lane : 0.f);
    z_h[g] = wave_sum((is_hi && g_col == g) ? z_lane : 0.f);
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
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (gq == 0 && g < G) wo[wave][g][ch] = v * sc + z_h[g];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = cpv[J][r];
        v += __shfl_xor(v, 32);
        const int g = 4 * (gq & 1) + r;
        const float zg = (gq & 1) ? z_h[4 + r] : z_h[r];
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
  finish_work_group<GP>(a, b, h, s, wm, wl, wo, qraw);
}

}  // namespace

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);

// Group sizes up to 8 run on the matrix cores; 9..16 query heads per KV head
// (two MFMA row blocks of hi/lo would not fit 16 rows) use the VALU kernel.
int launch_decode_mfma(const DecodeArgs& a, int batch, void* stream) {
  const int G = a.group;
  if (G > 8) return launch_decode_valu(a, batch, stream);
  dim3 grid(a.n_split, a.n_kv_heads, batch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (G <= 1) hipLaunchKernelGGL(decode_mfma_kernel<1>, grid, dim3(256), 0, st, a);
  else if (G <= 2) hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, dim3(256), 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_mfma_kernel<8>, grid, dim3(256), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
