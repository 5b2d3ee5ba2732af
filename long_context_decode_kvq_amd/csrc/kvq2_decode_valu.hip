// Split-K decode attention, plain VALU variant (fp32 FMA).
//
// Kept beside the MFMA kernel as the measured comparison point: at INT2 one
// HBM byte carries ~14 (G = 4) to ~28 (G = 8) useful multiply-adds, more than
// fp32 VALU can sustain at HBM speed, which the rocprofv3 numbers of the two
// kernels show side by side.
//
// Grid (n_split, Hkv, B); 256 threads = 4 waves.  Work-group s < n_split_int2
// walks INT2 chunks [c_begin, c_end) of (b, h), one 16-token chunk per wave
// per step; work-group n_split_int2 takes the bf16 sink and recent tokens.
//   QK:  lane (t = lane/4, quarter = lane%4) dots 32 channels of token t's
//        codes with q' (LDS), quad-reduced; logit = s_K*(q'.c) + z_K*sum(q').
//   PV:  lane owns channels 2*lane, 2*lane+1; o' += (p*s_V)*c, and the zero
//        term sum(p*z_V) is added to every channel at the end.
#include "kvq2_decode_common.h"

namespace kvq {
namespace {

template <int GP>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  __shared__ float qs[GP][kHeadDim];
  __shared__ float qsum[GP];
  __shared__ int qexp[GP];
  __shared__ float wbuf[4][16][GP];          // p * s_V of each token of the wave's chunk
  __shared__ float pbuf[4][16][GP];          // p of each bf16 token
  __shared__ float wm[4][GP], wl[4][GP];
  __shared__ float wo[4][GP][kHeadDim];
  __shared__ float cm[kCombineSlice][GP], cl[kCombineSlice][GP];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = a.seq_len[b];

  load_queries<GP>(a, b, h, qs, qsum, qexp);

  float m[GP], l[GP], zacc[GP], acc0[GP], acc1[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) { m[g] = -INFINITY; l[g] = 0.f; zacc[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }

  const int t = lane >> 2, qq = lane & 3;

  const Int2Range rg = int2_range(a, L, 1);
  if (s < a.n_split_int2) {
    int t_begin, t_end;
    split_tiles(a, rg, 1, s, t_begin, t_end);
    for (int c = rg.cf + t_begin + wave; c < rg.cf + t_end; c += 4) {
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, c * kChunkTokens);
      if (off < 0) continue;   // invalid page entry: the chunk is skipped
      const uint8_t* ch = a.pool + off;
      const uint2 kc = *reinterpret_cast<const uint2*>(ch + kKCodesOff + 32 * t + 8 * qq);
      const uint32_t kp = *reinterpret_cast<const uint32_t*>(ch + kKParamsOff + 4 * t);
      const uint32_t vp = *reinterpret_cast<const uint32_t*>(ch + kVParamsOff + 4 * t);
      float lg[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        float dot = 0.f;
        if (g < G) {
          const float* qv = &qs[g][32 * qq];
#pragma unroll
          for (int k = 0; k < 16; ++k) dot = fmaf(qv[k], float((kc.x >> (2 * k)) & 3u), dot);
#pragma unroll
          for (int k = 0; k < 16; ++k) dot = fmaf(qv[16 + k], float((kc.y >> (2 * k)) & 3u), dot);
        }
        dot += dpp_move<kQuadXor1>(dot);
        dot += dpp_move<kQuadXor2>(dot);
        const float sk = f16_bits_to_float(kp & 0xFFFFu), zk = f16_bits_to_float(kp >> 16);
        lg[g] = (g < G) ? fmaf(sk, dot, zk * qsum[g]) : -INFINITY;
      }
      float corr[GP];
      softmax_tile16<GP>(G, qq, lg, corr, m, l);
      const float sv = f16_bits_to_float(vp & 0xFFFFu);
      const float zv = f16_bits_to_float(vp >> 16);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (qq == 0) wbuf[wave][t][g] = lg[g] * sv;
        zacc[g] = zacc[g] * corr[g] + ((qq == 0) ? lg[g] * zv : 0.f);
        acc0[g] *= corr[g];
        acc1[g] *= corr[g];
      }
      __builtin_amdgcn_wave_barrier();
      // V codes of channel group gc = lane/2 for the 16 tokens: 4 dwords.
      const int gc = lane >> 1;
      const uint8_t* vb = ch + kVCodesOff + 32 * (gc & 15) + 4 * (gc >> 4);
      uint32_t vd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) vd[k] = *reinterpret_cast<const uint32_t*>(vb + 8 * k);
      const int sh = 4 * (lane & 1);
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const uint32_t byte = (vd[tt >> 2] >> (8 * (tt & 3))) & 0xFFu;
        const float c0 = float((byte >> sh) & 3u), c1 = float((byte >> (sh + 2)) & 3u);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float w = wbuf[wave][tt][g];
          acc0[g] = fmaf(w, c0, acc0[g]);
          acc1[g] = fmaf(w, c1, acc1[g]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    const TokenList tl = token_list(a, L, rg);
    for (int tile = wave; tile * 16 < tl.n_all; tile += 4)
      token_tile<GP>(a, b, h, tl, rg, tile, qs, qsum, pbuf[wave], m, l, acc0, acc1);
  }

  // Wave state -> LDS (o' = acc + zero term on every channel).
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const float zs = wave_sum(zacc[g]);
    if (g < G) {
      wo[wave][g][2 * lane] = acc0[g] + zs;
      wo[wave][g][2 * lane + 1] = acc1[g] + zs;
      if (lane == 0) { wm[wave][g] = m[g]; wl[wave][g] = l[g]; }
    }
  }
  __syncthreads();
  const int64_t head = int64_t(b) * a.n_kv_heads + h;
  finish_work_group<GP>(a, b, h, head * a.n_split + s, head * a.n_split, a.n_split, 0, 0, wm, wl,
                        wo, qs, cm, cl);
}

}  // namespace

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream) {
  dim3 grid(a.n_split, a.n_kv_heads, batch);
  const int G = a.group;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // G = 1 runs the two-head instantiation with one padding head.
  if (G <= 2) hipLaunchKernelGGL(decode_valu_kernel<2>, grid, dim3(256), 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL(decode_valu_kernel<4>, grid, dim3(256), 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL(decode_valu_kernel<8>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_valu_kernel<16>, grid, dim3(256), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
