// Grouped expert GEMMs with fp8 (OCP e4m3) operands and fp32 block scales, large-tile
// form: the fp8 counterpart of the bf16 128-row tiled kernel, for layers whose experts
// receive many rows (the DeepSeek-V3-like layer of an FFN instance aggregating
// attention batches; FP8/BF16 mixed precision: the omica.com.cn AFD article, §3.3).
//
// A workgroup of kFp8TiledWavesM x 4 waves computes a 128-row tile of one expert
// times 8 32-column groups; wave (m, n) owns rows m * 128 / WM .. and groups 2n, 2n+1.
// One reduction step is one 128-deep scale block, i.e. one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 block; its fp32 partial product is
// added times s_act[row][kb] * s_w[kb][nb].  Weight fragments (2 KiB: 64 lanes x 32
// bytes) stream from HBM straight into registers a few steps ahead; the 128 gathered
// activation rows (fp8 codes) and their per-row scales are staged through
// double-buffered LDS, chunk by chunk, shared by all waves.  Items and XCD ranges as
// in the bf16 tiled kernel.
#include "grouped.h"

namespace afd {

constexpr int kF8RowBlocks = 8;
constexpr int kF8Rows = 16 * kF8RowBlocks;  // 128
constexpr int kF8GroupsPerWave = 2;
constexpr int kF8WavesN = 4;
constexpr int kF8Groups = kF8WavesN * kF8GroupsPerWave;
#ifndef AFD_FP8_TILED_WAVES_M
#define AFD_FP8_TILED_WAVES_M 2
#endif
constexpr int kF8WavesM = AFD_FP8_TILED_WAVES_M;
constexpr int kF8Waves = kF8WavesM * kF8WavesN;
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8WaveRowBlocks = kF8RowBlocks / kF8WavesM;
constexpr int kF8StageBlocks = kF8RowBlocks / kF8Waves;
constexpr int kF8BAhead = 2;  // 128-deep weight steps in flight per wave (8 KiB each); the
                              // even/odd step loop below relies on this being 2
constexpr int kF8Chunk = 1;   // 128-deep steps per staged activation chunk
constexpr int kF8Xcds = 8;

struct Fp8TiledSmem {
  i32x8 a[2][kF8Chunk][kF8RowBlocks][kWave];  // [buffer][step][row block][lane] 32-byte fragments
  float s[2][kF8Chunk][kF8Rows];              // activation scales of the staged rows
};

__device__ __forceinline__ f32x4 f8_mfma(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

__device__ __forceinline__ i32x8 f8_load32(const uint8_t* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  const i32x4 lo = q[0], hi = q[1];
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kF8Threads, 1) gemm_fp8_tiled_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kF8Waves + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  Fp8TiledSmem& sm = *reinterpret_cast<Fp8TiledSmem*>(dyn_smem);

  const int total = build_item_prefix(g, kF8Rows, kF8Groups, prefix, scan_tmp);
  const int w = threadIdx.x / kWave;
  const int wm = w / kF8WavesN;
  const int wn = w % kF8WavesN;

  const int xcd = blockIdx.x % kF8Xcds;
  const int slot = blockIdx.x / kF8Xcds;
  const int slots = gridDim.x / kF8Xcds;
  const int begin = (int)((long long)total * xcd / kF8Xcds);
  const int end = (int)((long long)total * (xcd + 1) / kF8Xcds);

  for (int item = begin + slot; item < end; item += slots) {
    // Lane-derived indices are recomputed per item: hoisted out of the item loop they
    // (row indices and addresses of the epilogue) no longer fit the register budget.
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const Item it = decode_item_tiled(g, kF8Rows, kF8Groups, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 128;
    const int NC = (KB + kF8Chunk - 1) / kF8Chunk;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    const int N = groups * 32;
    const int NB = N / 128;
    // waves past the last group recompute valid groups and store nothing (even group
    // counts: group0 + 1 < groups)
    const bool active = it.group + wn * kF8GroupsPerWave < groups;
    const int group0 = active ? it.group + wn * kF8GroupsPerWave : groups - kF8GroupsPerWave;

    // staged rows of this lane (row blocks w * kF8StageBlocks + j), clamped into the tile
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const uint8_t* abase = static_cast<const uint8_t*>(it.shared ? g.a_shared : g.a_routed);
    const float* asbase = it.shared ? g.as_shared : g.as_routed;
    const uint8_t* arow[kF8StageBlocks];
#pragma unroll
    for (int j = 0; j < kF8StageBlocks; ++j) {
      int r = (w * kF8StageBlocks + j) * 16 + (lane & 15);
      r = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[j] = abase + (size_t)ar * lda + (lane >> 4) * 32;
    }
    // activation-scale row staged by this thread (threads 0..127: one tile row each)
    const float* srow = nullptr;
    if (threadIdx.x < kF8Rows) {
      int r = threadIdx.x < it.nrows ? threadIdx.x : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      srow = asbase + (size_t)ar * KB;
    }

    const uint8_t* wbase = it.shared ? static_cast<const uint8_t*>(g.w_shared)
                                     : static_cast<const uint8_t*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const size_t group_stride = (size_t)KB * 4096;  // bytes per 32-column group
    const uint8_t* B = wbase + (size_t)group0 * group_stride + lane * 32;
    const float* ws = it.shared ? g.s_shared : g.s_routed + (size_t)it.seg * g.s_expert_elems;
    int nbc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int j = group0 + (cb >> 1), half = cb & 1;
      nbc[cb] = (SWIGLU ? half * (N / 2) + j * 16 : j * 32 + half * 16) / 128;
    }

    f32x4 acc[kF8WaveRowBlocks][4];
#pragma unroll
    for (int rb = 0; rb < kF8WaveRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    i32x8 bring[kF8BAhead][4];
#pragma unroll
    for (int u = 0; u < kF8BAhead; ++u) {
      const int s = u < KB ? u : KB - 1;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) bring[u][cb] = f8_load32(B + (cb >> 1) * group_stride + (s * 2 + (cb & 1)) * 2048);
    }

    // activation chunk 0 -> LDS buffer 0, chunk 1 -> staging registers (steps past
    // the end of K repeat the last step; they are never consumed)
    i32x8 stage[kF8StageBlocks][kF8Chunk];
    float sstage[kF8Chunk];
#pragma unroll
    for (int u = 0; u < kF8Chunk; ++u) {
      const int s = u < KB ? u : KB - 1;
#pragma unroll
      for (int j = 0; j < kF8StageBlocks; ++j) stage[j][u] = f8_load32(arow[j] + s * 128);
      sstage[u] = srow ? srow[s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kF8Chunk; ++u) {
#pragma unroll
      for (int j = 0; j < kF8StageBlocks; ++j) sm.a[0][u][w * kF8StageBlocks + j][lane] = stage[j][u];
      if (srow) sm.s[0][u][threadIdx.x] = sstage[u];
    }
    if (NC > 1) {
#pragma unroll
      for (int u = 0; u < kF8Chunk; ++u) {
        int s = kF8Chunk + u;
        s = s < KB ? s : KB - 1;
#pragma unroll
        for (int j = 0; j < kF8StageBlocks; ++j) stage[j][u] = f8_load32(arow[j] + s * 128);
        sstage[u] = srow ? srow[s] : 0.f;
      }
    }
    __syncthreads();

    const int rsub = (lane >> 4) * 4;
    // One 128-deep step per LDS buffer and per weight-ring slot; the loop handles an
    // even and an odd step per iteration so that both indices are compile-time
    // constants (a runtime ring index put the ring in scratch memory).  A step past
    // the end of K recomputes the last step with weight scale 0 (no branch around the
    // MFMAs: see the bf16 tiled kernel).
    auto step = [&](const int c, const int par) {
      const int kbc = c < KB ? c : KB - 1;
      const float live = c < KB ? 1.f : 0.f;
      const i32x8* abuf = &sm.a[par][0][wm * kF8WaveRowBlocks][lane];
      const float* sbuf = &sm.s[par][0][wm * kF8WaveRowBlocks * 16 + rsub];
      float wsc[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) wsc[cb] = ws[(size_t)kbc * NB + nbc[cb]] * live;
#pragma unroll
      for (int rb = 0; rb < kF8WaveRowBlocks; ++rb) {
        const i32x8 a = abuf[rb * kWave];
        const f32x4 sa = *reinterpret_cast<const f32x4*>(sbuf + rb * 16);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const f32x4 p = f8_mfma(a, bring[par][cb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(p[i], sa[i] * wsc[cb], acc[rb][cb][i]);
        }
        // consume each row block's partial products before the next block's MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
      int sn = c + kF8BAhead;
      sn = sn < KB ? sn : KB - 1;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bring[par][cb] = f8_load32(B + (cb >> 1) * group_stride + (sn * 2 + (cb & 1)) * 2048);
      // stage the next step into the other buffer, then fetch the one after it
      if (c + 1 < NC) {
#pragma unroll
        for (int j = 0; j < kF8StageBlocks; ++j) sm.a[par ^ 1][0][w * kF8StageBlocks + j][lane] = stage[j][0];
        if (srow) sm.s[par ^ 1][0][threadIdx.x] = sstage[0];
      }
      __syncthreads();
      if (c + 2 < NC) {
        int s2 = c + 2;
        s2 = s2 < KB ? s2 : KB - 1;
#pragma unroll
        for (int j = 0; j < kF8StageBlocks; ++j) stage[j][0] = f8_load32(arow[j] + s2 * 128);
        sstage[0] = srow ? srow[s2] : 0.f;
      }
    };
    for (int c = 0; c < NC; c += 2) {
      step(c, 0);
      if (c + 1 < NC) step(c + 1, 1);
    }

    if (active) {
      const int col = lane & 15;
      const int rw0 = wm * kF8WaveRowBlocks * 16;
      float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
      const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
      for (int gi = 0; gi < kF8GroupsPerWave; ++gi)
#pragma unroll
        for (int rb = 0; rb < kF8WaveRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = rw0 + rb * 16 + rsub + i;
            if (row >= it.nrows) continue;
            float* o = out + (size_t)(it.row0 + row) * ldo;
            if (SWIGLU) {
              o[(group0 + gi) * 16 + col] = silu(acc[rb][2 * gi][i]) * acc[rb][2 * gi + 1][i];
            } else {
              o[(group0 + gi) * 32 + col] = acc[rb][2 * gi][i];
              o[(group0 + gi) * 32 + 16 + col] = acc[rb][2 * gi + 1][i];
            }
          }
    }
    __syncthreads();
  }
}

template <bool SWIGLU>
static hipError_t launch_fp8_tiled(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = sizeof(Fp8TiledSmem);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<SWIGLU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    configured = true;
  }
  long long blocks = max_items < max_blocks ? max_items : max_blocks;
  blocks = blocks < kF8Xcds ? kF8Xcds : blocks / kF8Xcds * kF8Xcds;
  gemm_fp8_tiled_kernel<SWIGLU><<<(unsigned)blocks, kF8Threads, smem, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                 hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  return swiglu ? launch_fp8_tiled<true>(g, max_items, max_blocks, st) : launch_fp8_tiled<false>(g, max_items, max_blocks, st);
}

}  // namespace afd
