// Grouped expert GEMMs in fp32 on the vector ALUs (the all-fp32 layer).
//
// Same work items as the bf16 kernels (16-row tile of one expert's rows times a
// 32-column group, statically strided over the waves), on weights in their natural
// row-major layout.  fp32 matrix-core throughput equals the fp32 vector peak on
// gfx950, so plain FMAs lose nothing here.  The reduction is split over the wave's
// four 16-lane groups: lane l owns column (l % 16) of each 16-column block and the
// reduction quarter l / 16, accumulating all 16 rows of the tile over its quarter (a
// quarter of the dependent steps of a whole-K walk, four times the work per step).
// The four partial sums are then added across the lane groups in a fixed order,
// (q0 + q1) + (q2 + q3), and lanes 0..15 store the tile.
#include "grouped.h"

namespace afd {

constexpr int kF32Threads = 256;
constexpr int kF32Waves = kF32Threads / kWave;
constexpr int kF32Ahead = 2;  // 4-step groups of the reduction in flight per lane

template <bool SWIGLU>
__global__ void __launch_bounds__(kF32Threads) gemm_f32_kernel(GroupedGemm g) {
  __shared__ SegTable prefix;
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
    const int q = lane >> 4;            // reduction quarter
    const int KQ = K / 4;               // K is a multiple of 128
    const int k0 = q * KQ;
    // the tile's 16 rows (rows past the tile end repeat its first row; not stored)
    const float* arow[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const int rr = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + rr;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + rr] / g.k : it.row0 + rr;
      arow[r] = Abase + (size_t)ar * lda + k0;
    }
    // weights [K][N] row-major; N = 2 * (groups * 16) for gate/up, groups * 32 for down
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    const int N = groups * 32;
    const float* W = (it.shared ? static_cast<const float*>(g.w_shared)
                                : static_cast<const float*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems) +
                     (size_t)k0 * N;
    const int col0 = SWIGLU ? it.group * 16 + c : it.group * 32 + c;
    const int col1 = SWIGLU ? N / 2 + it.group * 16 + c : it.group * 32 + 16 + c;
    // loads run two 4-step groups ahead in a rotating register ring (each row's 4
    // activations of a group in one 16-byte load); the FMAs of each quarter keep
    // ascending k order
    float acc0[kTileRows], acc1[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) acc0[r] = acc1[r] = 0.f;
    float w0r[kF32Ahead][4], w1r[kF32Ahead][4];
    float4 ar[kF32Ahead][kTileRows];
    auto load = [&](int kk, int u) {  // steps kk .. kk + 3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0r[u][i] = W[(size_t)(kk + i) * N + col0];
        w1r[u][i] = W[(size_t)(kk + i) * N + col1];
      }
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) ar[u][r] = *reinterpret_cast<const float4*>(arow[r] + kk);
    };
#pragma unroll
    for (int u = 0; u < kF32Ahead; ++u) load(4 * u, u);
    for (int kb = 0; kb < KQ; kb += 4 * kF32Ahead) {
#pragma unroll
      for (int u = 0; u < kF32Ahead; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < kTileRows; ++r) {
            const float av = i == 0 ? ar[u][r].x : i == 1 ? ar[u][r].y : i == 2 ? ar[u][r].z : ar[u][r].w;
            acc0[r] = fmaf(av, w0r[u][i], acc0[r]);
            acc1[r] = fmaf(av, w1r[u][i], acc1[r]);
          }
        const int kn = kb + 4 * (kF32Ahead + u);
        load(kn < KQ ? kn : KQ - 4, u);  // past the end: reload the last group, unused
      }
    }
    // (q0 + q1) + (q2 + q3): the same sum, bit for bit, in every lane of the column
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      acc0[r] += __shfl_xor(acc0[r], 16, kWave);
      acc1[r] += __shfl_xor(acc1[r], 16, kWave);
      acc0[r] += __shfl_xor(acc0[r], 32, kWave);
      acc1[r] += __shfl_xor(acc1[r], 32, kWave);
    }
    if (q == 0) {
      float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
      const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
      for (int r = 0; r < kTileRows; ++r) {
        if (r >= it.nrows) continue;
        float* o = out + (size_t)(it.row0 + r) * ldo;
        if (SWIGLU) {
          o[it.group * 16 + c] = silu(acc0[r]) * acc1[r];
        } else {
          o[it.group * 32 + c] = acc0[r];
          o[it.group * 32 + 16 + c] = acc1[r];
        }
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
