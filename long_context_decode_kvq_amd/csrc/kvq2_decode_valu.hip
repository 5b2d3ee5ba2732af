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
  __shared__ float qraw[GP][kHeadDim];
  __shared__ float qs[GP][kHeadDim];
  __shared__ float qsum[GP];
  __shared__ float wbuf[4][16][GP];          // p * s_V of each token of the wave's chunk
  __shared__ float pbuf[4][16][GP];          // p of each bf16 token
  __shared__ float wm[4][GP], wl[4][GP];
  __shared__ float wo[4][GP][kHeadDim];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = a.seq_len[b];

  rotate_queries<GP>(a, b, h, qraw, qs, qsum);

  float m[GP], l[GP], zacc[GP], acc0[GP], acc1[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) { m[g] = -INFINITY; l[g] = 0.f; zacc[g] = 0.f; acc0[g] = 0.f; acc1[g] = 0.f; }

  const int t = lane >> 2, qq = lane & 3;
  // Online-softmax update for one 16-token tile whose per-lane logits are in
  // `lg` (lane (t, qq) holds token t; -inf for masked tokens).  Returns the
  // correction factor per head and leaves p in `lg`.
  auto softmax_tile = [&](float* lg, float* corr) {
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
      const float p = exp2f(lg[g] - mn);
      float ps = (qq == 0) ? p : 0.f;
      ps = wave_sum(ps);
      l[g] = l[g] * corr[g] + ps;
      m[g] = mn;
      lg[g] = p;
    }
  };

  if (s < a.n_split_int2) {
    int c_begin, c_end, int2_end;
    int2_chunk_range(a, L, s, c_begin, c_end, int2_end);
    for (int c = c_begin + wave; c < c_end; c += 4) {
      const int pos = c * kChunkTokens + t;
      const int64_t off = chunk_offset(a.block_table, a.bt_stride, a.num_pages, a.n_kv_heads,
                                       a.page_size, b, h, c * kChunkTokens);
      if (off < 0) continue;   // invalid page entry: the chunk is skipped
      const uint8_t* ch = a.pool + off;
      const bool valid = pos >= a.n_sink && pos < int2_end;
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
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const float sk = f16_bits_to_float(kp & 0xFFFFu), zk = f16_bits_to_float(kp >> 16);
        lg[g] = valid ? fmaf(sk, dot, zk * qsum[g]) : -INFINITY;
      }
      float corr[GP];
      softmax_tile(lg, corr);
      const float sv = valid ? f16_bits_to_float(vp & 0xFFFFu) : 0.f;
      const float zv = valid ? f16_bits_to_float(vp >> 16) : 0.f;
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
    // bf16 sink and recent tokens, in tiles of 16 per wave.
    const int n_sk = min(L, a.n_sink);
    const int r_begin = max(a.n_sink, L - a.n_recent);
    const int n_bf = n_sk + max(0, L - r_begin);
    const int64_t sh_base = int64_t(b) * a.n_kv_heads + h;
    auto token_ptr = [&](int idx) -> const uint16_t* {
      const int pos = idx < n_sk ? idx : r_begin + (idx - n_sk);
      if (pos < a.n_sink) return a.sink + (sh_base * a.n_sink + pos) * 2 * kHeadDim;
      return a.recent + (sh_base * a.n_recent + (pos - a.n_sink) % a.n_recent) * 2 * kHeadDim;
    };
    for (int tile = wave; tile * 16 < n_bf; tile += 4) {
      const int idx = tile * 16 + t;
      const bool valid = idx < n_bf;
      float lg[GP];
      const uint16_t* kp = token_ptr(valid ? idx : 0) + 32 * qq;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        float dot = 0.f;
        if (g < G && valid) {
#pragma unroll
          for (int k = 0; k < 32; ++k) dot = fmaf(qs[g][32 * qq + k], bf16_bits_to_float(kp[k]), dot);
        }
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        lg[g] = valid ? dot : -INFINITY;
      }
      float corr[GP];
      softmax_tile(lg, corr);
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (qq == 0) pbuf[wave][t][g] = lg[g];
        acc0[g] *= corr[g];
        acc1[g] *= corr[g];
      }
      __builtin_amdgcn_wave_barrier();
      const int nt = min(16, n_bf - tile * 16);
      for (int tt = 0; tt < nt; ++tt) {
        const uint32_t v2 = *reinterpret_cast<const uint32_t*>(token_ptr(tile * 16 + tt) + kHeadDim + 2 * lane);
        const float v0 = bf16_bits_to_float(v2 & 0xFFFFu), v1 = bf16_bits_to_float(v2 >> 16);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float p = pbuf[wave][tt][g];
          acc0[g] = fmaf(p, v0, acc0[g]);
          acc1[g] = fmaf(p, v1, acc1[g]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
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
  finish_work_group<GP>(a, b, h, s, wm, wl, wo, qraw);
}

}  // namespace

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream) {
  dim3 grid(a.n_split, a.n_kv_heads, batch);
  const int G = a.group;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (G <= 1) hipLaunchKernelGGL(decode_valu_kernel<1>, grid, dim3(256), 0, st, a);
  else if (G <= 2) hipLaunchKernelGGL(decode_valu_kernel<2>, grid, dim3(256), 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL(decode_valu_kernel<4>, grid, dim3(256), 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL(decode_valu_kernel<8>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_valu_kernel<16>, grid, dim3(256), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
