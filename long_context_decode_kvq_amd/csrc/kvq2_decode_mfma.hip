// Launch side of the matrix-core decode (kernels in kvq2_decode_mfma_kernels.h):
// the per-device launch geometry, the range cut's weights and the launches.
// The kernels of quantization groups narrower than the head are built in
// kvq2_decode_mfma_groups.hip, those of eight query heads per KV head in
// kvq2_decode_mfma_g8.hip and those of decodes with shared-prefix groups in
// kvq2_decode_mfma_prefix.hip (separate code objects).
#include <algorithm>
#include <mutex>

#include "kvq2_decode_mfma_kernels.h"

namespace kvq {

int launch_decode_valu(const DecodeArgs& a, int batch, void* stream);
// kvq2_decode_mfma_groups.hip: the kernels of narrower quantization groups
int decode_mfma_groups_per_cu(int gp, int ng);
int launch_decode_mfma_groups(const DecodeArgs& a, unsigned grid, void* stream);
// kvq2_decode_mfma_g8.hip: the kernels of eight query heads per KV head
int decode_mfma_g8_per_cu();
void launch_decode_mfma_g8(const DecodeArgs& a, unsigned grid, bool per_head, void* stream);
// kvq2_decode_mfma_prefix.hip: the kernels of decodes with shared-prefix groups
void launch_decode_mfma_prefix(const DecodeArgs& a, unsigned grid, bool per_head, void* stream);

// Group sizes up to 8 run on the matrix cores; 9..16 query heads per KV head
// (two MFMA row blocks of hi/lo would not fit 16 rows) use the VALU kernel.
namespace {

// Per-device launch geometry, queried once per device: compute units and
// the work-groups of each decode kernel one CU holds at once.
struct DeviceGeometry {
  int cus;
  // decode_mfma_kernel<2, ng>, <4, ng> for ng = 1, 2, 4; <8, 1>
  int per_cu[3][3];
};

template <int GP, int NG>
int kernel_per_cu() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_kernel<GP, NG>, 256, 0) !=
          hipSuccess || per_cu <= 0)
    return 1;
  return per_cu;
}

constexpr int ng_index(int ng) { return ng == 1 ? 0 : ng == 2 ? 1 : 2; }

const DeviceGeometry& device_geometry() {
  constexpr int kMaxDevices = 64;
  static DeviceGeometry cached[kMaxDevices];
  static std::once_flag once[kMaxDevices];
  static const DeviceGeometry fallback = {256, {{1, 1, 1}, {1, 1, 1}, {1, 1, 1}}};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fallback;
  std::call_once(once[dev], [dev] {
    DeviceGeometry g = fallback;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      g.cus = cus;
    g.per_cu[0][0] = kernel_per_cu<2, 1>();
    g.per_cu[0][1] = decode_mfma_groups_per_cu(2, 2);
    g.per_cu[0][2] = decode_mfma_groups_per_cu(2, 4);
    g.per_cu[1][0] = kernel_per_cu<4, 1>();
    g.per_cu[1][1] = decode_mfma_groups_per_cu(4, 2);
    g.per_cu[1][2] = decode_mfma_groups_per_cu(4, 4);
    g.per_cu[2][0] = g.per_cu[2][1] = g.per_cu[2][2] = decode_mfma_g8_per_cu();
    cached[dev] = g;
  });
  return cached[dev];
}

int device_cus() { return device_geometry().cus; }

template <int GP, int NG>
int resident_work_groups() {
  const DeviceGeometry& g = device_geometry();
  return g.cus * g.per_cu[GP == 2 ? 0 : GP == 4 ? 1 : 2][ng_index(NG)];
}

// Work-groups of the equal-range decode: one round of resident work-groups,
// but no more than one per kMinTilesPerGroup tiles (bounded above from
// max_seq_len), so that short or few sequences are not cut into pieces whose
// fixed cost (prologue, partial, combine) dominates -- yet one per CU while
// each still gets kMinTilesPerCuGroup tiles, so that small batches fill the
// GPU (measured at batch 1: 32768 tokens 46.8 -> 37.4 us per step with 256
// work-groups instead of 64; more than one round of small ranges was slower).
// 64 tiles per work-group: one sequence of 131072 tokens (32768 tiles over 8
// KV heads) decodes in 40.5 us with 512 work-groups, 47.5 us with 256 (128
// tiles each) and 52.7 us with 1024 (32 tiles each).
constexpr int kMinTilesPerGroup = 64;
constexpr int kMinTilesPerCuGroup = 32;

template <int GP, int NG>
int chain_grid(const DecodeArgs& a, int batch, int max_seq_len) {
  constexpr int NPT = Geo<GP, NG>::NPT;
  const int64_t int2_end = std::max<int64_t>(a.n_sink, int64_t(max_seq_len) - a.n_recent);
  const int64_t tiles = std::max<int64_t>(1, (int2_end / kChunkTokens) / NPT);
  const int64_t est = int64_t(batch) * a.n_kv_heads * tiles;
  const int64_t cus = std::max(1, device_cus());
  const int64_t want = std::max<int64_t>(
      (est + kMinTilesPerGroup - 1) / kMinTilesPerGroup,
      std::min<int64_t>(cus, est / kMinTilesPerCuGroup));
  return int(std::max<int64_t>(
      1, std::min<int64_t>(want, std::min(kChainGroups, resident_work_groups<GP, NG>()))));
}

}  // namespace

// Grid and range weights of the MFMA decode (before the pre-pass, which
// writes the cut): one round of resident work-groups, each range weighted by
// its work-group's dispatch round and XCD (decode_tuning()).
void set_chain_geometry(DecodeArgs& a, int batch, int max_seq_len) {
  const int G = a.group;
  const int ng = a.ng;
  if (G <= 2)
    a.chain_groups = ng == 1 ? chain_grid<2, 1>(a, batch, max_seq_len)
                   : ng == 2 ? chain_grid<2, 2>(a, batch, max_seq_len)
                             : chain_grid<2, 4>(a, batch, max_seq_len);
  else if (G <= 4)
    a.chain_groups = ng == 1 ? chain_grid<4, 1>(a, batch, max_seq_len)
                   : ng == 2 ? chain_grid<4, 2>(a, batch, max_seq_len)
                             : chain_grid<4, 4>(a, batch, max_seq_len);
  else
    a.chain_groups = chain_grid<8, 1>(a, batch, max_seq_len);
  a.round_size = device_cus();
  const DecodeTuning& t = decode_tuning();
  const int k = G > 4 ? 1 : 0;
  for (int r = 0; r < 4; ++r) a.round_weight[r] = t.round_weight[k][r];
  for (int x = 0; x < 8; ++x) a.xcd_weight[x] = t.xcd_weight[k][x & 1];
}

int launch_decode_mfma(const DecodeArgs& a, int batch, int max_seq_len, void* stream) {
  const int G = a.group;
  if (G > 8) return launch_decode_valu(a, batch, stream);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)batch;
  (void)max_seq_len;
  // G = 1 runs the two-head kernel with one padding head.
  // the streaming work-groups, then one per token-list slice of every (b, h)
  const dim3 grid(a.chain_groups + a.batch * a.n_kv_heads * a.n_tok_slices);
  const bool per_head = 2 * a.batch * a.n_kv_heads < std::max(1, device_cus());
  const dim3 cgrid(a.n_kv_heads, a.batch, per_head ? a.group : 1);
  const dim3 cblock(per_head ? 128 * kHeadCombineParts
                             : (a.gp == 2 ? combine_threads<2>() : combine_threads<4>()));
  if (a.n_groups > 0) {
    launch_decode_mfma_prefix(a, grid.x, per_head, stream);
  } else if (G <= 2) {
    if (a.ng == 1) hipLaunchKernelGGL((decode_mfma_kernel<2, 1>), grid, dim3(256), 0, st, a);
    else launch_decode_mfma_groups(a, grid.x, stream);
    if (per_head) hipLaunchKernelGGL(combine_head_kernel<2>, cgrid, cblock, 0, st, a);
    else hipLaunchKernelGGL(combine_kernel<2>, cgrid, cblock, 0, st, a);
  } else if (G <= 4) {
    if (a.ng == 1) hipLaunchKernelGGL((decode_mfma_kernel<4, 1>), grid, dim3(256), 0, st, a);
    else launch_decode_mfma_groups(a, grid.x, stream);
    if (per_head) hipLaunchKernelGGL(combine_head_kernel<4>, cgrid, cblock, 0, st, a);
    else hipLaunchKernelGGL(combine_kernel<4>, cgrid, cblock, 0, st, a);
  } else {
    launch_decode_mfma_g8(a, grid.x, per_head, stream);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace kvq
