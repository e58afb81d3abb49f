// Grouped expert GEMMs in bf16 on the gfx950 matrix cores, large-tile form, for
// batches where experts receive many tokens (an FFN instance aggregating several
// attention instances' batches: "大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §2, and the MegaScale-Infer summary in "AF分离论文串讲").
//
// A workgroup of 4 waves computes a 128-row tile of one expert's rows times 8
// 32-column groups; wave w owns groups 2w and 2w+1 (4 16-column blocks) for all 128
// rows, i.e. 8 x 4 accumulators of v_mfma_f32_16x16x32_bf16.  Each weight fragment
// is used by exactly one wave, so weights stream straight from HBM into registers
// (fragment order, 4 reduction steps ahead, as in the weight-streaming kernel); the
// 128 gathered activation rows are shared by the 4 waves and staged through LDS in
// MFMA A-operand order, one K-chunk at a time, double-buffered: the next chunk's
// global loads are issued before the current chunk is consumed.
//
// Items are (segment, column tile, row tile) with the row tile fastest, and the item
// list is cut into 8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8):
// the row tiles of a hot expert and the neighbouring column tiles run at the same
// time on one XCD and share its L2 for the weights and the activation rows.
#include "grouped.h"

namespace afd {

constexpr int kTiledRowBlocks = 8;                      // 16-row blocks per tile
constexpr int kTiledRows = 16 * kTiledRowBlocks;        // 128
constexpr int kTiledGroupsPerWave = 2;                  // 32-column groups per wave
constexpr int kTiledWavesN = 4;                         // waves across the columns
constexpr int kTiledGroups = kTiledWavesN * kTiledGroupsPerWave;  // per item
#ifndef AFD_TILED_WAVES_M
#define AFD_TILED_WAVES_M 1
#endif
constexpr int kTiledWavesM = AFD_TILED_WAVES_M;         // waves across the rows (1 or 2)
constexpr int kTiledWaves = kTiledWavesM * kTiledWavesN;
constexpr int kTiledThreads = kTiledWaves * kWave;
constexpr int kTiledWaveRowBlocks = kTiledRowBlocks / kTiledWavesM;  // row blocks per wave
constexpr int kTiledStageBlocks = kTiledRowBlocks / kTiledWaves;     // row blocks each wave stages
#ifndef AFD_TILED_B_AHEAD
#define AFD_TILED_B_AHEAD 4
#endif
constexpr int kTiledBAhead = AFD_TILED_B_AHEAD;         // weight steps in flight per wave
constexpr int kXcds = 8;

template <int KC>
struct TiledSmem {
  // [buffer][step in chunk][row block][lane] 16-byte A fragments
  bf16x8 a[2][KC][kTiledRowBlocks][kWave];
};

#ifndef AFD_TILED_B_NT
#define AFD_TILED_B_NT 0
#endif
__device__ __forceinline__ bf16x8 tiled_load_b(const i32x4* p) {
#if AFD_TILED_B_NT
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(p));
#else
  return __builtin_bit_cast(bf16x8, *p);
#endif
}

template <bool SWIGLU, int KC>
__global__ void __launch_bounds__(kTiledThreads, 1) gemm_bf16_tiled_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kTiledWaves + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  TiledSmem<KC>& sm = *reinterpret_cast<TiledSmem<KC>*>(dyn_smem);

  const int total = build_item_prefix(g, kTiledRows, kTiledGroups, prefix, scan_tmp);
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int wm = w / kTiledWavesN;  // row half of this wave
  const int wn = w % kTiledWavesN;  // column quarter of this wave

  // XCD-aware striding: this workgroup's XCD owns a contiguous range of items
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int begin = (int)((long long)total * xcd / kXcds);
  const int end = (int)((long long)total * (xcd + 1) / kXcds);

  for (int item = begin + slot; item < end; item += slots) {
    const Item it = decode_item_tiled(g, kTiledRows, kTiledGroups, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 32;
    const int NC = KB / KC;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    // First group of this wave.  A wave past the last group of a partial column tile
    // recomputes the tile's last two groups and stores nothing: the main loop stays
    // free of branches, which keeps the accumulators in place (a branch around the
    // MFMAs made the compiler copy all of them through VGPRs every chunk).  Group
    // counts are even (multiples of 128 columns), so group0 + 1 < groups.
    const bool active = it.group + wn * kTiledGroupsPerWave < groups;  // wave-uniform
    const int group0 = active ? it.group + wn * kTiledGroupsPerWave : groups - kTiledGroupsPerWave;

    // this lane's staged A rows (row blocks w * kTiledStageBlocks + j), clamped
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const __bf16* abase = static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed);
    const bf16x8* arow[kTiledStageBlocks];
#pragma unroll
    for (int j = 0; j < kTiledStageBlocks; ++j) {
      int r = (w * kTiledStageBlocks + j) * 16 + (lane & 15);
      r = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[j] = reinterpret_cast<const bf16x8*>(abase + (size_t)ar * lda) + (lane >> 4);
    }
    // weights of this wave: groups group0, group0 + 1, each [KB][2 halves][64 lanes]
    const __bf16* wbase = it.shared ? static_cast<const __bf16*>(g.w_shared)
                                    : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const i32x4* B = reinterpret_cast<const i32x4*>(wbase) + (size_t)group0 * KB * 128 + lane;
    const size_t group_stride = (size_t)KB * 128;

    f32x4 acc[kTiledWaveRowBlocks][4];
#pragma unroll
    for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // weight ring: step s lives in slot s % kTiledBAhead
    bf16x8 bring[kTiledBAhead][4];
#pragma unroll
    for (int u = 0; u < kTiledBAhead; ++u)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bring[u][cb] = tiled_load_b(B + (cb >> 1) * group_stride + (u * 2 + (cb & 1)) * 64);

    // A chunk 0 -> LDS buffer 0, chunk 1 -> staging registers
    bf16x8 stage[kTiledStageBlocks][KC];
#pragma unroll
    for (int u = 0; u < KC; ++u)
#pragma unroll
      for (int j = 0; j < kTiledStageBlocks; ++j) stage[j][u] = arow[j][u * 4];
#pragma unroll
    for (int u = 0; u < KC; ++u)
#pragma unroll
      for (int j = 0; j < kTiledStageBlocks; ++j) sm.a[0][u][w * kTiledStageBlocks + j][lane] = stage[j][u];
    if (NC > 1) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int j = 0; j < kTiledStageBlocks; ++j) stage[j][u] = arow[j][(KC + u) * 4];
    }
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
      const int buf = c & 1;
#pragma unroll
      for (int u = 0; u < KC; ++u) {
        const int slotb = u % kTiledBAhead;
        bf16x8 a[kTiledWaveRowBlocks];
#pragma unroll
        for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb) a[rb] = sm.a[buf][u][wm * kTiledWaveRowBlocks + rb][lane];
#pragma unroll
        for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], bring[slotb][cb], acc[rb][cb], 0, 0, 0);
        // refill this ring slot with the step kTiledBAhead ahead (clamped to the last)
        int s = c * KC + u + kTiledBAhead;
        s = s < KB ? s : KB - 1;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          bring[slotb][cb] = tiled_load_b(B + (cb >> 1) * group_stride + (s * 2 + (cb & 1)) * 64);
      }
      if (c + 1 < NC) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int j = 0; j < kTiledStageBlocks; ++j) sm.a[buf ^ 1][u][w * kTiledStageBlocks + j][lane] = stage[j][u];
      }
      __syncthreads();
      if (c + 2 < NC) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int j = 0; j < kTiledStageBlocks; ++j) stage[j][u] = arow[j][((c + 2) * KC + u) * 4];
      }
    }

    if (active) {
      const int col = lane & 15;
      const int rsub = (lane >> 4) * 4;
      const int rw0 = wm * kTiledWaveRowBlocks * 16;  // first tile row of this wave
      if (SWIGLU) {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int gi = 0; gi < kTiledGroupsPerWave; ++gi)
#pragma unroll
          for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = rw0 + rb * 16 + rsub + i;
              if (row < it.nrows)
                out[(size_t)(it.row0 + row) * ldo + (group0 + gi) * 16 + col] =
                    f32_to_bf16(silu(acc[rb][2 * gi][i]) * acc[rb][2 * gi + 1][i]);
            }
      } else {
        float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int gi = 0; gi < kTiledGroupsPerWave; ++gi)
#pragma unroll
          for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = rw0 + rb * 16 + rsub + i;
              if (row < it.nrows) {
                float* o = out + (size_t)(it.row0 + row) * ldo + (group0 + gi) * 32 + col;
                o[0] = acc[rb][2 * gi][i];
                o[16] = acc[rb][2 * gi + 1][i];
              }
            }
      }
    }
    // the next item's first LDS writes must not overtake this item's last reads
    __syncthreads();
  }
}

template <bool SWIGLU, int KC>
static hipError_t launch_tiled(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = sizeof(TiledSmem<KC>);
  static bool configured = false;  // raise the dynamic LDS limit once per process
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_tiled_kernel<SWIGLU, KC>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    configured = true;
  }
  long long blocks = max_items < max_blocks ? max_items : max_blocks;
  blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
  gemm_bf16_tiled_kernel<SWIGLU, KC><<<(unsigned)blocks, kTiledThreads, smem, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                  hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  // 4-step (128-deep) activation chunks: every K here is a multiple of 128, and an
  // 8-step chunk's staging registers spill
  return swiglu ? launch_tiled<true, 4>(g, max_items, max_blocks, st) : launch_tiled<false, 4>(g, max_items, max_blocks, st);
}

int tiled_rows() { return kTiledRows; }
int tiled_groups() { return kTiledGroups; }

}  // namespace afd
