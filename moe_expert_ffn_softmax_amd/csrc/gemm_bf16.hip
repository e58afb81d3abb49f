// Grouped expert GEMMs in bf16 on the gfx950 matrix cores, weight-streaming form.
//
// The expert FFN's dominant cost is reading expert weights that only a few tokens
// use ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §1: each expert's weight
// matrices are large but a step activates them with few tokens; MoE FFN utilisation
// falls from 28% at batch 395 to 0.5% at batch 6).  This kernel is built for that
// regime: one wave computes a 16-row tile (the tokens of one expert, padded) times
// 32 output columns over the whole reduction, streaming that column group's
// pre-packed weight fragments straight from HBM into registers: every lane issues
// 16-byte loads that together cover contiguous 1 KiB fragments, two fragments per
// 32-deep step, loaded eight steps ahead of use (nontemporal), and each fragment feeds one
// v_mfma_f32_16x16x32_bf16 directly (no LDS round trip: each weight byte is used by
// exactly one wave).  The 16 activation rows of the tile are gathered through the
// expert-sorted pair order (tokens of x for the gate/up projection, intermediate
// rows for the down projection).
//
//   gate/up (SWIGLU = true): the column group holds gate block j and up block j, so
//     the epilogue forms h = SiLU(gate) * up in registers and stores bf16 h;
//   down    (SWIGLU = false): the group holds output blocks 2j and 2j+1, stored as
//     bf16 rows for the combine (which sums them in fp32).
// MFMA operand order (16x16x32 bf16): lane l supplies row (l % 16) of A and column
// (l % 16) of B at reduction offsets (l / 16) * 8 .. + 7; it receives rows
// (l / 16) * 4 .. + 3 of column (l % 16) of the 16x16 fp32 result.
#include "grouped.h"

namespace afd {

constexpr int kGemmThreads = 256;
constexpr int kGemmWaves = kGemmThreads / kWave;

// Weight fragments are read exactly once per launch: load them nontemporally so they
// stream past the caches instead of evicting the activation rows every wave re-reads.
__device__ __forceinline__ bf16x8 load_weight_frag(const i32x4* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(p));
}

// acc0/acc1 += A[16 x K] * B[K x 32] over K = 32 * KB, with the loads of step s + D
// issued while step s computes (a rotating register pipeline; no branch inside, so
// the compiler waits only for the oldest outstanding loads).  KB % D == 0, KB >= D.
template <int D>
__device__ __forceinline__ void stream_mfma(const bf16x8* __restrict__ A, const i32x4* __restrict__ B, int KB,
                                            f32x4& acc0, f32x4& acc1) {
  bf16x8 a[D], b0[D], b1[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    a[u] = A[u * 4];
    b0[u] = load_weight_frag(B + (u * 2) * 64);
    b1[u] = load_weight_frag(B + (u * 2 + 1) * 64);
  }
  for (int s0 = D; s0 < KB; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
      const int s = s0 + u;
      a[u] = A[s * 4];
      b0[u] = load_weight_frag(B + (s * 2) * 64);
      b1[u] = load_weight_frag(B + (s * 2 + 1) * 64);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
  }
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kGemmThreads) gemm_bf16_stream_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kGemmWaves + 1];
  const int total = build_item_prefix(g, kTileRows, prefix, scan_tmp);
  const int lane = lane_id();
  const int waves_in_launch = gridDim.x * kGemmWaves;
  const int wave = blockIdx.x * kGemmWaves + threadIdx.x / kWave;

  for (int item = wave; item < total; item += waves_in_launch) {
    const Item it = decode_item(g, kTileRows, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 32;
    // A row of this lane (rows past the tile end repeat its first row; their
    // results are not stored)
    const int r = lane & 15;
    const int rr = r < it.nrows ? r : 0;
    int arow;
    if (it.shared)
      arow = it.row0 + rr;
    else
      arow = g.gather_routed ? g.sorted_pair[it.row0 + rr] / g.k : it.row0 + rr;
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const bf16x8* A = reinterpret_cast<const bf16x8*>(
                          static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed) + (size_t)arow * lda) +
                      (lane >> 4);
    const __bf16* wbase = it.shared ? static_cast<const __bf16*>(g.w_shared)
                                    : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const i32x4* B = reinterpret_cast<const i32x4*>(wbase) + (size_t)it.group * KB * 128 + lane;

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (KB % 8 == 0)
      stream_mfma<8>(A, B, KB, acc0, acc1);
    else
      stream_mfma<4>(A, B, KB, acc0, acc1);

    const int col = lane & 15;
    const int rbase = (lane >> 4) * 4;
    if (SWIGLU) {
      __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
      const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + i;
        if (row < it.nrows)
          out[(size_t)(it.row0 + row) * ldo + it.group * 16 + col] = f32_to_bf16(silu(acc0[i]) * acc1[i]);
      }
    } else {
      __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
      const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + i;
        if (row < it.nrows) {
          __bf16* o = out + (size_t)(it.row0 + row) * ldo + it.group * 32 + col;
          o[0] = f32_to_bf16(acc0[i]);
          o[16] = f32_to_bf16(acc1[i]);
        }
      }
    }
  }
}

hipError_t launch_gemm_bf16(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  // persistent grid of resident workgroups only: a workgroup that waits for a free
  // slot would start its items a whole item late
  long long blocks = (max_items + kGemmWaves - 1) / kGemmWaves;
  if (blocks > max_blocks) blocks = max_blocks;
  if (swiglu)
    gemm_bf16_stream_kernel<true><<<(unsigned)blocks, kGemmThreads, 0, st>>>(g);
  else
    gemm_bf16_stream_kernel<false><<<(unsigned)blocks, kGemmThreads, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace afd

namespace afd {
hipError_t gemm_occupancy_bf16(int* gate_up, int* down) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(gate_up, gemm_bf16_stream_kernel<true>, kGemmThreads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(down, gemm_bf16_stream_kernel<false>, kGemmThreads, 0);
  return e;
}
}  // namespace afd
