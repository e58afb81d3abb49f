// Grouped expert GEMMs in fp32 on the vector ALUs (the all-fp32 layer).
//
// Same work items as the bf16 kernels (16-row tile of one expert's rows times a
// 32-column group, statically strided over the waves), on weights in their natural
// row-major layout.  fp32 matrix-core throughput equals the fp32 vector peak on
// gfx950, so plain FMAs lose nothing here.  Lane l owns column (l % 16) of each
// 16-column block and rows (l / 16) * 4 .. + 3 of the tile.
#include "grouped.h"

namespace afd {

constexpr int kF32Threads = 256;
constexpr int kF32Waves = kF32Threads / kWave;
constexpr int kF32Ahead = 8;  // reduction steps in flight

template <bool SWIGLU>
__global__ void __launch_bounds__(kF32Threads) gemm_f32_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kF32Waves + 1];
  const int total = build_item_prefix(g, kTileRows, prefix, scan_tmp);
  const int lane = lane_id();
  const int waves_in_launch = gridDim.x * kF32Waves;
  const int wave = blockIdx.x * kF32Waves + threadIdx.x / kWave;

  for (int item = wave; item < total; item += waves_in_launch) {
    const Item it = decode_item(g, kTileRows, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const float* Abase = static_cast<const float*>(it.shared ? g.a_shared : g.a_routed);
    const int c = lane & 15;
    const int rbase = (lane >> 4) * 4;
    const float* arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + i < it.nrows ? rbase + i : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[i] = Abase + (size_t)ar * lda;
    }
    // weights [K][N] row-major; N = 2 * (groups * 16) for gate/up, groups * 32 for down
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    const int N = groups * 32;
    const float* W = it.shared ? static_cast<const float*>(g.w_shared)
                               : static_cast<const float*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const int col0 = SWIGLU ? it.group * 16 + c : it.group * 32 + c;
    const int col1 = SWIGLU ? N / 2 + it.group * 16 + c : it.group * 32 + 16 + c;
    // loads run kF32Ahead reduction steps ahead in a rotating register ring (K is a
    // multiple of 128); the FMAs keep ascending k order
    float acc0[4] = {0.f, 0.f, 0.f, 0.f}, acc1[4] = {0.f, 0.f, 0.f, 0.f};
    float w0r[kF32Ahead], w1r[kF32Ahead], ar[kF32Ahead][4];
    auto load = [&](int kk, int u) {
      w0r[u] = W[(size_t)kk * N + col0];
      w1r[u] = W[(size_t)kk * N + col1];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[u][i] = arow[i][kk];
    };
#pragma unroll
    for (int u = 0; u < kF32Ahead; ++u) load(u, u);
    for (int k0 = 0; k0 < K; k0 += kF32Ahead) {
#pragma unroll
      for (int u = 0; u < kF32Ahead; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[i] = fmaf(ar[u][i], w0r[u], acc0[i]);
          acc1[i] = fmaf(ar[u][i], w1r[u], acc1[i]);
        }
        const int kn = k0 + kF32Ahead + u;
        load(kn < K ? kn : K - 1, u);  // past the end: reload the last step, unused
      }
    }
    float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
    const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rbase + i;
      if (row >= it.nrows) continue;
      float* o = out + (size_t)(it.row0 + row) * ldo;
      if (SWIGLU) {
        o[it.group * 16 + c] = silu(acc0[i]) * acc1[i];
      } else {
        o[it.group * 32 + c] = acc0[i];
        o[it.group * 32 + 16 + c] = acc1[i];
      }
    }
  }
}

hipError_t launch_gemm_f32(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  long long blocks = (max_items + kF32Waves - 1) / kF32Waves;
  if (blocks > max_blocks) blocks = max_blocks;
  if (swiglu)
    gemm_f32_kernel<true><<<(unsigned)blocks, kF32Threads, 0, st>>>(g);
  else
    gemm_f32_kernel<false><<<(unsigned)blocks, kF32Threads, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace afd

namespace afd {
hipError_t gemm_occupancy_f32(int* gate_up, int* down) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(gate_up, gemm_f32_kernel<true>, kF32Threads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(down, gemm_f32_kernel<false>, kF32Threads, 0);
  return e;
}
}  // namespace afd
