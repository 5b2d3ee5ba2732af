// Self-test of libkvq2's host code under the address and undefined-behaviour
// sanitizers (built with tests/host_sanitize/launch_stubs.cpp in place of the
// HIP launchers): every public entry point's validation, the decode planning
// over a sweep of shapes, and the host calibration on seeded bf16 data.
// Prints "host selftest ok" and exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "kvq2.h"
#include "kvq2_hqmq.h"
#include "kvq2_internal.h"

namespace kvq {
extern int g_launches;
extern size_t g_last_ws_bytes;
}

static int g_fail = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

int main() {
  // fake, 16-byte aligned device addresses: validation must never touch them
  auto fake = [](uintptr_t off) { return reinterpret_cast<void*>(uintptr_t(0x7F0000000000) + off); };
  kvq_dims d = {32, 8, 128, 16, 4, 256, 0.0f};
  kvq_layer lay = {static_cast<const float*>(fake(0)), static_cast<const float*>(fake(0x100000)),
                   4.0f, 4.0f};
  kvq_cache c = {static_cast<uint8_t*>(fake(0x200000)), 100,
                 static_cast<uint16_t*>(fake(0x300000)), static_cast<uint16_t*>(fake(0x400000)),
                 static_cast<const int32_t*>(fake(0x500000)), 64};
  const int32_t* i32 = static_cast<const int32_t*>(fake(0x600000));
  const uint16_t* u16 = static_cast<const uint16_t*>(fake(0x700000));
  float* f32 = static_cast<float*>(fake(0x800000));
  void* ws = fake(0x900000);

  for (int s : {0, -1, -2, -3, -4, -5, -99}) CHECK(std::strncmp(kvq_status_string(s), "KVQ_", 4) == 0);
  CHECK(kvq_last_error() != nullptr);

  // ---- validation: every error before any launch
  const int before = kvq::g_launches;
  kvq_dims bad = d;
  bad.head_dim = 64;
  CHECK(kvq_decode_attention(&bad, &lay, &c, 2, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_UNSUPPORTED);
  CHECK(kvq_decode_attention_noalloc(&bad, &lay, &c, 2, i32, 100, u16, f32, nullptr) == KVQ_ERR_UNSUPPORTED);
  CHECK(kvq_quantize_append(&bad, &lay, &c, 2, i32, i32, 4, 2, u16, u16, nullptr) == KVQ_ERR_UNSUPPORTED);
  bad = d;
  bad.n_q_heads = 34;
  CHECK(kvq_decode_attention(&bad, &lay, &c, 2, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(nullptr, &lay, &c, 2, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(&d, nullptr, &c, 2, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(&d, &lay, nullptr, 2, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(&d, &lay, &c, 2, i32, 100, u16 + 1, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(&d, &lay, &c, 2, i32, 64 * 16 + 1, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_decode_attention(&d, &lay, &c, 2, i32, 100, u16, f32, ws, 16, nullptr) == KVQ_ERR_WORKSPACE);
  CHECK(kvq_decode_step(&d, &lay, &c, 2, i32, i32, 4, 5, u16, u16, i32, 100, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_quantize_append(&d, &lay, &c, 2, i32, i32, 4, 2, u16 + 4, u16, nullptr) == KVQ_ERR_ARG);
  kvq_layer nan_clip = lay;
  nan_clip.clip_V = std::nanf("");
  CHECK(kvq_quantize_append(&d, &nan_clip, &c, 2, i32, i32, 4, 2, u16, u16, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq::g_launches == before);

  // ---- valid calls reach the launchers with the planned workspace
  const size_t need = kvq_decode_workspace_bytes(&d, 2, 100);
  CHECK(need > 0);
  CHECK(kvq_decode_attention(&d, &lay, &c, 2, i32, 100, u16, f32, ws, need, nullptr) == KVQ_OK);
  CHECK(kvq::g_last_ws_bytes == need);
  CHECK(kvq_decode_attention_noalloc(&d, &lay, &c, 2, i32, 100, u16, f32, nullptr) == KVQ_OK);
  CHECK(kvq_decode_step(&d, &lay, &c, 2, i32, i32, 2, 1, u16, u16, i32, 100, u16, f32, ws, need, nullptr) == KVQ_OK);
  CHECK(kvq_quantize_append(&d, &lay, &c, 2, i32, i32, 0, 0, nullptr, nullptr, nullptr) == KVQ_OK);

  // ---- multi-query attention: 1 <= M <= n_recent, passes of at most 8 rows
  const size_t need4 = kvq_decode_multi_workspace_bytes(&d, 2, 100, 4);
  const size_t need2 = kvq_decode_multi_workspace_bytes(&d, 2, 100, 2);
  CHECK(need2 > need);                                  // 8 rows: more partials
  CHECK(need4 == need2);                                // 16 rows: two passes of 8
  CHECK(kvq_decode_multi_workspace_bytes(&d, 2, 100, 1) == need);
  const int before_multi = kvq::g_launches;
  CHECK(kvq_decode_multi_attention(&d, &lay, &c, 2, i32, 100, 5, u16, f32, ws, need4, nullptr) == KVQ_OK);
  CHECK(kvq::g_launches == before_multi + 3);           // queries 0-1, 2-3, 4
  CHECK(kvq_decode_multi_attention(&d, &lay, &c, 2, i32, 100, 4, u16, f32, ws, need4 - 1, nullptr) == KVQ_ERR_WORKSPACE);
  CHECK(kvq_decode_multi_attention(&d, &lay, &c, 2, i32, 100, 0, u16, f32, ws, need4, nullptr) == KVQ_ERR_ARG);
  kvq_dims w2 = d;
  w2.n_recent = 2;
  CHECK(kvq_decode_multi_attention(&w2, &lay, &c, 2, i32, 100, 3, u16, f32, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);

  // ---- prefix-aware decode: groups validated, their workspace planned
  {
    kvq_prefix_groups g = {1, 2, i32, i32, i32};
    const size_t needp = kvq_decode_prefix_workspace_bytes(&d, 2, 100, &g);
    CHECK(needp > need);
    const int before_prefix = kvq::g_launches;
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, &g, ws, needp, nullptr) == KVQ_OK);
    CHECK(kvq::g_launches == before_prefix + 1);
    CHECK(kvq::g_last_ws_bytes == needp);
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, &g, ws, needp - 1, nullptr) == KVQ_ERR_WORKSPACE);
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, nullptr, ws, needp, nullptr) == KVQ_ERR_ARG);
    kvq_prefix_groups bad = {257, 2, i32, i32, i32};
    CHECK(kvq_decode_prefix_workspace_bytes(&d, 2, 100, &bad) == 0);
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, &bad, ws, needp, nullptr) == KVQ_ERR_ARG);
    kvq_prefix_groups none = {0, 0, nullptr, nullptr, nullptr};
    CHECK(kvq_decode_prefix_workspace_bytes(&d, 2, 100, &none) == need);
    kvq_prefix_groups null_arrays = {1, 2, nullptr, i32, i32};
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, &null_arrays, ws, needp, nullptr) == KVQ_ERR_ARG);
    // member counts large enough to overflow the 32-bit virtual tile count
    // the row-set items' tiles overflow the 32-bit virtual tile count
    kvq_prefix_groups big = {256, 1024, i32, i32, i32};
    kvq_cache long_c = c;
    long_c.bt_stride = 1 << 18;
    CHECK(kvq_decode_prefix_attention(&d, &lay, &long_c, 2, i32, 1 << 22, u16, f32, &big, ws, size_t(1) << 40, nullptr) == KVQ_ERR_UNSUPPORTED);
    kvq_prefix_groups too_many = {256, 1025, i32, i32, i32};
    CHECK(kvq_decode_prefix_workspace_bytes(&d, 2, 100, &too_many) == 0);
    CHECK(kvq_decode_prefix_attention(&d, &lay, &c, 2, i32, 100, u16, f32, &too_many, ws, 1 << 30, nullptr) == KVQ_ERR_ARG);
  }

  // ---- planning over a sweep of shapes (no overflow, monotone in batch)
  for (int G : {1, 2, 3, 4, 8, 16})
    for (int P : {16, 32, 64})
      for (int W : {1, 128, 8192}) {
        kvq_dims s = {8 * G, 8, 128, P, 4, W, 0.0f};
        size_t prev = 0;
        for (int B : {1, 7, 64, 512}) {
          const size_t b = kvq_decode_workspace_bytes(&s, B, 131072);
          CHECK(b >= prev);
          prev = b;
        }
      }

  // ---- host calibration on seeded data
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int N : {1, 17, 64}) {
    const int Hq = 4, Hkv = 2;
    std::vector<uint16_t> q(N * Hq * 128), k(N * Hkv * 128), v(N * Hkv * 128);
    for (auto& x : q) x = bf16(nd(rng));
    for (auto& x : k) x = bf16(2.f * nd(rng));
    for (auto& x : v) x = bf16(nd(rng));
    std::vector<float> RK(Hkv * 128 * 128), RV(RK.size());
    float cK = 0, cV = 0;
    kvq_dims s = {Hq, Hkv, 128, 16, 4, 128, 0.0f};
    CHECK(kvq_calibrate(&s, N, q.data(), k.data(), v.data(), 0.999, RK.data(), RV.data(), &cK, &cV) == KVQ_OK);
    CHECK(cK > 0 && cV > 0);
    double worst = 0;   // R^T R = I
    for (int h = 0; h < Hkv; ++h)
      for (int i = 0; i < 128; ++i)
        for (int j = 0; j < 128; ++j) {
          double dot = 0;
          for (int r = 0; r < 128; ++r)
            dot += double(RK[(h * 128 + r) * 128 + i]) * RK[(h * 128 + r) * 128 + j];
          worst = std::fmax(worst, std::fabs(dot - (i == j)));
        }
    CHECK(worst < 1e-5);
    q[3] = 0x7F80;   // +inf
    CHECK(kvq_calibrate(&s, N, q.data(), k.data(), v.data(), 0.999, RK.data(), RV.data(), &cK, &cV) == KVQ_ERR_NUMERIC);
    CHECK(kvq_calibrate(&s, N, q.data(), k.data(), v.data(), 1.5, RK.data(), RV.data(), &cK, &cV) == KVQ_ERR_ARG);
  }
  // ---- HQMQ codec: validation, planning, the host codebook product
  {
    kvq_hqmq_dims hd = {32, 8, 128, 16, 10, 0.0f};
    kvq_hqmq_layer hl = {static_cast<const float*>(fake(0)), static_cast<const float*>(fake(0x1000))};
    kvq_hqmq_cache hc = {static_cast<uint8_t*>(fake(0x200000)), 100,
                         static_cast<const int32_t*>(fake(0x300000)), 8};
    const size_t aws = kvq_hqmq_append_workspace_bytes(&hd, 100);
    CHECK(aws > 0);
    const int32_t* ip = static_cast<const int32_t*>(fake(0x400000));
    const uint16_t* up = static_cast<const uint16_t*>(fake(0x500000));
    const int before = kvq::g_launches;
    CHECK(kvq_hqmq_append(&hd, &hl, &hc, 2, ip, ip, 4, 2, up, up, fake(0x600000), aws, nullptr) == KVQ_OK);
    CHECK(kvq::g_launches == before + 1);
    CHECK(kvq_hqmq_append(&hd, &hl, &hc, 2, ip, ip, 4, 2, up, up, fake(0x600000), aws - 1, nullptr) == KVQ_ERR_WORKSPACE);
    CHECK(kvq_hqmq_append(&hd, &hl, &hc, 2, ip, ip, 0, 0, nullptr, nullptr, nullptr, 0, nullptr) == KVQ_OK);
    for (int B : {1, 7, 64, 65535})
      for (int L : {0, 1, 255, 4096, 131072, 1 << 30}) {
        const size_t need = kvq_hqmq_decode_workspace_bytes(&hd, B, L);
        CHECK(need > 0);
        CHECK(kvq_hqmq_decode_attention(&hd, &hl, &hc, B, ip, L, up, static_cast<float*>(fake(0x700000)),
                                        fake(0x800000), need, nullptr) == KVQ_OK);
        CHECK(kvq::g_last_ws_bytes == need);
      }
    for (int G : {1, 4, 5, 8, 16}) {
      kvq_hqmq_dims g = {8 * G, 8, 128, 64, 3, 0.0f};
      CHECK(kvq_hqmq_decode_workspace_bytes(&g, 3, 1000) > 0);
    }
    kvq_hqmq_dims bad = hd;
    bad.n_secondary = 11;
    CHECK(kvq_hqmq_decode_workspace_bytes(&bad, 1, 10) == 0);
    float sec[40], cb[960];
    std::mt19937 r2(7);
    for (float& x : sec) x = nd(r2);
    for (int S = 1; S <= 10; ++S) CHECK(kvq_hqmq_codebook(S, sec, cb) == KVQ_OK);
    CHECK(kvq_hqmq_codebook(0, sec, cb) == KVQ_ERR_ARG);
    sec[5] = NAN;
    CHECK(kvq_hqmq_codebook(4, sec, cb) == KVQ_ERR_NUMERIC);
  }
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host selftest ok\n");
  return 0;
}
