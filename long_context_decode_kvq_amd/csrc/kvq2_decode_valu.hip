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
//        codes with q' (LDS); each lane adds its channels' share
//        s_K*(q'.c) + z_K*sum(q') with the (s_K, z_K) of their quantization
//        group, and the quad sum is the logit.
//   PV:  lane owns channels 2*lane, 2*lane+1 and dequantizes them with the
//        (s_V, z_V) of their group: o' += p*(s_V*c + z_V).
// Quantization groups of 128, 64 or 32 channels (one, two or four (s, z)
// pairs per vector) share the code layout; only the parameter offsets and
// the chunk size differ.
#include "kvq2_decode_common.h"

namespace kvq {
namespace {

template <int GP>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  __shared__ float qs[GP][kHeadDim];
  __shared__ float qsum[GP];
  __shared__ float qsum4[GP][4];             // sum(q') over channels 32 k .. 32 k + 31
  __shared__ int qexp[GP];
  __shared__ float wbuf[4][16][GP];          // p of each token of the wave's chunk
  __shared__ float pbuf[4][16][GP];          // p of each bf16 token
  __shared__ float wm[4][GP], wl[4][GP];
  __shared__ float wo[4][GP][kHeadDim];
  __shared__ float cm[kCombineSlice][GP], cl[kCombineSlice][GP];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = a.seq_len[b];

  load_queries<GP>(a, b, h, qs, qsum, qexp);
  if (threadIdx.x < G * 4) {
    const int g = threadIdx.x >> 2, k = threadIdx.x & 3;
    float sum = 0.f;
    for (int c = 0; c < 32; ++c) sum += qs[g][32 * k + c];
    qsum4[g][k] = sum;
  }
  __syncthreads();

  float m[GP], l[GP], acc0[GP], acc1[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) { m[g] = -INFINITY; l[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }

  const int t = lane >> 2, qq = lane & 3;
  const int ng = a.ng;
  // quantization group of this lane's 32 key channels (32 qq ..) and of its
  // two value channels (2 lane, 2 lane + 1)
  const int kgrp = (qq * ng) >> 2, vgrp = (lane * ng) >> 6;

  const Int2Range rg = int2_range(a, L, 1);
  if (s < a.n_split_int2) {
    int t_begin, t_end;
    split_tiles(a, rg, 1, s, t_begin, t_end);
    for (int c = rg.cf + t_begin + wave; c < rg.cf + t_end; c += 4) {
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, c * kChunkTokens, a.chunk_bytes);
      if (off < 0) continue;   // invalid page entry: the chunk is skipped
      const uint8_t* ch = a.pool + off;
      const uint2 kc = *reinterpret_cast<const uint2*>(ch + kKCodesOff + 32 * t + 8 * qq);
      const uint32_t kp = *reinterpret_cast<const uint32_t*>(ch + param_offset(0, t, ng, kgrp));
      // (s_V, z_V) of this lane's value group for every token of the chunk
      uint32_t vps[16];
#pragma unroll
      for (int tt = 0; tt < 16; ++tt)
        vps[tt] = *reinterpret_cast<const uint32_t*>(ch + param_offset(1, tt, ng, vgrp));
      const float sk = f16_bits_to_float(kp & 0xFFFFu), zk = f16_bits_to_float(kp >> 16);
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
        // this lane's share of the logit: its group's s_K times its 32
        // channels' dot, plus z_K times their sum of q' (dequantization folded)
        float part = g < G ? fmaf(sk, dot, zk * qsum4[g][qq]) : 0.f;
        part += dpp_move<kQuadXor1>(part);
        part += dpp_move<kQuadXor2>(part);
        lg[g] = (g < G) ? part : -INFINITY;
      }
      float corr[GP];
      softmax_tile16<GP>(G, qq, lg, corr, m, l);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (qq == 0) wbuf[wave][t][g] = lg[g];
        acc0[g] *= corr[g];
        acc1[g] *= corr[g];
      }
      __builtin_amdgcn_wave_barrier();
      // V codes of channel group gc = lane/2 for the 16 tokens: 4 dwords;
      // each value dequantized with its group's (s_V, z_V)
      const int gc = lane >> 1;
      const uint8_t* vb = ch + kVCodesOff + 32 * (gc & 15) + 4 * (gc >> 4);
      uint32_t vd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) vd[k] = *reinterpret_cast<const uint32_t*>(vb + 8 * k);
      const int sh = 4 * (lane & 1);
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const uint32_t byte = (vd[tt >> 2] >> (8 * (tt & 3))) & 0xFFu;
        const float sv = f16_bits_to_float(vps[tt] & 0xFFFFu), zv = f16_bits_to_float(vps[tt] >> 16);
        const float v0 = fmaf(sv, float((byte >> sh) & 3u), zv);
        const float v1 = fmaf(sv, float((byte >> (sh + 2)) & 3u), zv);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float p = wbuf[wave][tt][g];
          acc0[g] = fmaf(p, v0, acc0[g]);
          acc1[g] = fmaf(p, v1, acc1[g]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
    const TokenList tl = token_list(a, L, rg);
    for (int tile = wave; tile * 16 < tl.n_all; tile += 4)
      token_tile<GP>(a, b, h, tl, rg, tile, qs, qsum, qsum4, pbuf[wave], m, l, acc0, acc1);
  }

  // Wave state -> LDS.
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < G) {
      wo[wave][g][2 * lane] = acc0[g];
      wo[wave][g][2 * lane + 1] = acc1[g];
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
