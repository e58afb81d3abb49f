// Grouped expert GEMMs in bf16 on the gfx950 matrix cores, large-tile form, for
// batches where experts receive many tokens (an FFN instance aggregating several
// attention instances' batches: "大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §2, and the MegaScale-Infer summary in "AF分离论文串讲").
//
// A workgroup of 4 waves computes a 128-row tile of one expert's rows times 8
// 32-column groups; wave w owns groups 2w and 2w+1, i.e. two 32x32 output blocks for
// every 32-row block: 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16.  (Measured on
// MI355X, the 32x32x16 form sustains ~2.2 PFLOP/s and the 16x16x32 form ~1.3.)
// Each weight fragment is used by exactly one wave, so weights stream from memory
// straight into registers, 4 reduction steps ahead; the 128 gathered activation rows
// are shared by the 4 waves and staged through LDS in MFMA A-operand order, one
// 128-deep chunk at a time, double-buffered: the next chunk's global loads are issued
// before the current chunk is consumed.
//
// Operands of the 32x32x16 MFMA: lane l supplies row (l % 32) of A and column (l % 32)
// of B at reduction offsets (l / 32) * 8 .. + 7 of the 16-deep step; it receives rows
// (i / 4) * 8 + (l / 32) * 4 + i % 4 (i = 0..15) of column (l % 32).  A lane's B data
// (8 consecutive reduction rows of one column) is one 16-byte chunk of the packed
// weight layout (see pack.hip), so a fragment is four 256-byte runs of it.
//
// SwiGLU pairing: for the gate/up projection a wave's two 32-column blocks are the
// gate and the up columns of the same 32 intermediate channels (groups 2w, 2w+1,
// gate halves, then up halves), so h = SiLU(gate) * up pairs values held by the same
// lane.  For the down projection the blocks are the wave's two groups.
//
// Items are (segment, column tile, row tile) with the row tile fastest, and the item
// list is cut into 8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8):
// the row tiles of a hot expert and the neighbouring column tiles run at the same
// time on one XCD and share its L2 for the weights and the activation rows.
#include "grouped.h"

namespace afd {

typedef float f32x16v __attribute__((ext_vector_type(16)));

#ifndef AFD_TILED_WAVES_M
#define AFD_TILED_WAVES_M 1
#endif
constexpr int kTiledWavesM = AFD_TILED_WAVES_M;         // waves across the rows (1 or 2)
constexpr int kTiledWavesN = 4;                         // waves across the columns
constexpr int kTiledWaves = kTiledWavesM * kTiledWavesN;
constexpr int kTiledThreads = kTiledWaves * kWave;
constexpr int kTiledRowBlocks = 4;                      // 32-row blocks per tile
constexpr int kTiledRows = 32 * kTiledRowBlocks;        // 128
constexpr int kTiledWaveRowBlocks = kTiledRowBlocks / kTiledWavesM;
constexpr int kTiledStage = kTiledRowBlocks * 2 / kTiledWaves;  // (row block, half) A fragments each wave stages
constexpr int kTiledGroupsPerWave = 2;                  // 32-column groups per wave
constexpr int kTiledGroups = kTiledWavesN * kTiledGroupsPerWave;  // per item
#ifndef AFD_TILED_B_AHEAD
#define AFD_TILED_B_AHEAD 4
#endif
constexpr int kTiledBAhead = AFD_TILED_B_AHEAD;         // 32-deep weight steps in flight per wave
constexpr int kXcds = 8;

template <int KC>
struct TiledSmem {
  // [buffer][32-deep step in chunk][16-deep half][row block][lane] 16-byte A fragments
  bf16x8 a[2][KC][2][kTiledRowBlocks][kWave];
};

__device__ __forceinline__ bf16x8 tiled_load_b(const bf16x8* p) { return *p; }

#ifndef AFD_TILED_MIN_BLOCKS
#define AFD_TILED_MIN_BLOCKS 2
#endif
constexpr int kTiledMinBlocks = AFD_TILED_MIN_BLOCKS;   // workgroups per CU the registers must allow

template <bool SWIGLU, int KC>
__global__ void __launch_bounds__(kTiledThreads, kTiledMinBlocks) gemm_bf16_tiled_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kTiledWaves + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  TiledSmem<KC>& sm = *reinterpret_cast<TiledSmem<KC>*>(dyn_smem);

  const int total = build_item_prefix(g, kTiledRows, kTiledGroups, prefix, scan_tmp);
  const int w = threadIdx.x / kWave;
  const int wm = w / kTiledWavesN;  // row part of this wave
  const int wn = w % kTiledWavesN;  // column part of this wave

  // XCD-aware striding: this workgroup's XCD owns a contiguous range of items
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int slots = gridDim.x / kXcds;
  const int begin = (int)((long long)total * xcd / kXcds);
  const int end = (int)((long long)total * (xcd + 1) / kXcds);

  for (int item = begin + slot; item < end; item += slots) {
    // lane-derived indices are recomputed per item (hoisted out of the item loop
    // they do not fit the register budget)
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const Item it = decode_item_tiled(g, kTiledRows, kTiledGroups, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 32;
    const int NC = KB / KC;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    // First group of this wave.  A wave past the last group of a partial column tile
    // recomputes the tile's last two groups and stores nothing: the main loop stays
    // free of branches around the MFMAs (such a branch made the compiler copy every
    // accumulator through VGPRs).  Group counts are even, so group0 + 1 < groups.
    const bool active = it.group + wn * kTiledGroupsPerWave < groups;  // wave-uniform
    const int group0 = active ? it.group + wn * kTiledGroupsPerWave : groups - kTiledGroupsPerWave;

    // A fragments this wave stages: (row block, half) pairs w * kTiledStage + j, as
    // row block = pair / 2, half = pair % 2; the lane's row is clamped into the tile
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const __bf16* abase = static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed);
    const bf16x8* arow[kTiledStage];
#pragma unroll
    for (int j = 0; j < kTiledStage; ++j) {
      const int pair = w * kTiledStage + j;
      int r = (pair >> 1) * 32 + (lane & 31);
      r = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[j] = reinterpret_cast<const bf16x8*>(abase + (size_t)ar * lda) + (lane >> 5) + (pair & 1) * 2;
    }
    // weights: 16-byte chunk of (step s, half kh) for block cb at bbase[cb] + s*128 + kh*32
    const __bf16* wbase = it.shared ? static_cast<const __bf16*>(g.w_shared)
                                    : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const bf16x8* bbase[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int grp = SWIGLU ? group0 + ((lane & 31) >> 4) : group0 + cb;
      const int half = SWIGLU ? cb : ((lane & 31) >> 4);
      bbase[cb] = reinterpret_cast<const bf16x8*>(wbase) + (size_t)grp * KB * 128 + half * 64 + (lane >> 5) * 16 +
                  (lane & 15);
    }

    f32x16v acc[kTiledWaveRowBlocks][2];
#pragma unroll
    for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = f32x16v{};

    // weight ring: step s lives in slot s % kTiledBAhead ([cb][kh])
    bf16x8 bring[kTiledBAhead][2][2];
#pragma unroll
    for (int u = 0; u < kTiledBAhead; ++u)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) bring[u][cb][kh] = tiled_load_b(bbase[cb] + u * 128 + kh * 32);

    // A chunk 0 -> LDS buffer 0, chunk 1 -> staging registers
    bf16x8 stage[KC][kTiledStage];
#pragma unroll
    for (int u = 0; u < KC; ++u)
#pragma unroll
      for (int j = 0; j < kTiledStage; ++j) stage[u][j] = arow[j][u * 4];
#pragma unroll
    for (int u = 0; u < KC; ++u)
#pragma unroll
      for (int j = 0; j < kTiledStage; ++j) {
        const int pair = w * kTiledStage + j;
        sm.a[0][u][pair & 1][pair >> 1][lane] = stage[u][j];
      }
    if (NC > 1) {
#pragma unroll
      for (int u = 0; u < KC; ++u)
#pragma unroll
        for (int j = 0; j < kTiledStage; ++j) stage[u][j] = arow[j][(KC + u) * 4];
    }
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
      const int buf = c & 1;
#pragma unroll
      for (int u = 0; u < KC; ++u) {
        const int slotb = u % kTiledBAhead;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          bf16x8 a[kTiledWaveRowBlocks];
#pragma unroll
          for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
            a[rb] = sm.a[buf][u][kh][wm * kTiledWaveRowBlocks + rb][lane];
#pragma unroll
          for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], bring[slotb][cb][kh], acc[rb][cb], 0, 0, 0);
        }
        // refill this ring slot with the step kTiledBAhead ahead (clamped to the last)
        int s = c * KC + u + kTiledBAhead;
        s = s < KB ? s : KB - 1;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) bring[slotb][cb][kh] = tiled_load_b(bbase[cb] + s * 128 + kh * 32);
      }
      if (c + 1 < NC) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int j = 0; j < kTiledStage; ++j) {
            const int pair = w * kTiledStage + j;
            sm.a[buf ^ 1][u][pair & 1][pair >> 1][lane] = stage[u][j];
          }
      }
      __syncthreads();
      if (c + 2 < NC) {
#pragma unroll
        for (int u = 0; u < KC; ++u)
#pragma unroll
          for (int j = 0; j < kTiledStage; ++j) stage[u][j] = arow[j][((c + 2) * KC + u) * 4];
      }
    }

    if (active) {
      const int col = lane & 31;
      const int rsub = (lane >> 5) * 4 + wm * kTiledWaveRowBlocks * 32;
      if (SWIGLU) {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < it.nrows)
              out[(size_t)(it.row0 + row) * ldo + group0 * 16 + col] =
                  f32_to_bf16(silu(acc[rb][0][i]) * acc[rb][1][i]);
          }
      } else {
        float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kTiledWaveRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < it.nrows) {
              float* o = out + (size_t)(it.row0 + row) * ldo + group0 * 32 + col;
              o[0] = acc[rb][0][i];
              o[32] = acc[rb][1][i];
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
  // max_blocks counts compute units; the kernel is built to keep kTiledMinBlocks
  // workgroups resident on each
  const long long resident = (long long)max_blocks * kTiledMinBlocks;
  long long blocks = max_items < resident ? max_items : resident;
  blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
  gemm_bf16_tiled_kernel<SWIGLU, KC><<<(unsigned)blocks, kTiledThreads, smem, st>>>(g);
  return hipGetLastError();
}

#ifndef AFD_TILED_KC
#define AFD_TILED_KC 4
#endif
hipError_t launch_gemm_bf16_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                  hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  // AFD_TILED_KC 32-deep steps per staged activation chunk when every reduction
  // length allows it, else 4 (every K here is a multiple of 128)
  constexpr int kc = AFD_TILED_KC;
  const bool big = (g.K_routed / 32) % kc == 0 && (g.shared_rows == 0 || (g.K_shared / 32) % kc == 0);
  if (big && kc != 4)
    return swiglu ? launch_tiled<true, kc>(g, max_items, max_blocks, st) : launch_tiled<false, kc>(g, max_items, max_blocks, st);
  return swiglu ? launch_tiled<true, 4>(g, max_items, max_blocks, st) : launch_tiled<false, 4>(g, max_items, max_blocks, st);
}

int tiled_rows() { return kTiledRows; }
int tiled_groups() { return kTiledGroups; }

}  // namespace afd
