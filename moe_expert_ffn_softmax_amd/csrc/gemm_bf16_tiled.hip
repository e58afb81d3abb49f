// Grouped expert GEMMs in bf16 on the gfx950 matrix cores, large-tile form, for
// batches where experts receive many tokens (an FFN instance aggregating several
// attention instances' batches: "大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §2, and the MegaScale-Infer summary in "AF分离论文串讲").
//
// A workgroup of 4 waves computes a 128-row tile of one expert's rows times 4 * GPW
// 32-column groups; wave w owns groups w*GPW .. +GPW-1, i.e. GPW 32x32 output blocks
// for every 32-row block: 4 x GPW accumulators of v_mfma_f32_32x32x16_bf16 (GPW = 2
// by default; 4 halves the weight traffic per FLOP but measured slower on these
// layers).  (Measured on MI355X, the 32x32x16 form sustains ~2.2 PFLOP/s on constant
// operands, ~1.75 on random ones, and the 16x16x32 form ~1.3.)
// Each weight fragment is used by exactly one wave, so weights stream from memory
// straight into registers, 8 / GPW reduction steps ahead; the 128 gathered activation rows
// are shared by the 4 waves and staged through LDS, one 128-deep chunk at a time,
// double-buffered.
//
// Activation staging.  The vector-memory path of a CU moves ~64 B/clk when each
// instruction reads a few long runs, but only ~16 B/clk when it reads 32 B from each
// of 32 rows.  So a wave loads its 32 rows of a chunk as 4 rows x 256 contiguous
// bytes per instruction (lane l: row l / 16, 16-byte piece l % 16) and rearranges
// them into MFMA operand order on the way into LDS.  LDS holds, per buffer, 4 row
// blocks x 8 fragments (16-deep halves of the 4 32-deep steps); a fragment keeps
// lane l' (row l' % 32, reduction half l' / 32) at byte (l' % 32) * 16 + (l' / 32) *
// 528 of a 1056-byte slot.  With that padding the 16 lanes writing one row (16
// different fragments and halves) hit 16 different 16-byte bank groups, and each
// 16-lane quarter of a fragment read is contiguous.
//
// Operands of the 32x32x16 MFMA: lane l supplies row (l % 32) of A and column (l % 32)
// of B at reduction offsets (l / 32) * 8 .. + 7 of the 16-deep step; it receives rows
// (i / 4) * 8 + (l / 32) * 4 + i % 4 (i = 0..15) of column (l % 32).  A lane's B data
// (8 consecutive reduction rows of one column) is one 16-byte chunk of the packed
// weight layout (see pack.hip), so a fragment is four 256-byte runs of it.
//
// SwiGLU pairing: for the gate/up projection the wave's 32-column blocks 2p and 2p+1
// are the gate and the up columns of the same 32 intermediate channels (gate halves,
// then up halves, of groups w*GPW + 2p and + 2p + 1), so h = SiLU(gate) * up pairs
// values held by the same lane.  For the down projection block cb is group w*GPW + cb.
//
// Items are (segment, column tile, row tile) with the row tile fastest, and the item
// list is cut into 8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8):
// the row tiles of a hot expert and the neighbouring column tiles run at the same
// time on one XCD and share its L2 for the weights and the activation rows.
#include "grouped.h"

namespace afd {

typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int kTiledWaves = 4;
constexpr int kTiledThreads = kTiledWaves * kWave;
constexpr int kTiledRowBlocks = 4;                      // 32-row blocks per tile (one per staging wave)
constexpr int kTiledRows = 32 * kTiledRowBlocks;        // 128
#ifndef AFD_TILED_GPW
#define AFD_TILED_GPW 2
#endif
constexpr int kTiledGroupsPerWave = AFD_TILED_GPW;      // 32-column groups per wave (2 or 4)
constexpr int kTiledGroups = kTiledWaves * kTiledGroupsPerWave;  // per item
static_assert(kTiledGroupsPerWave == 2 || kTiledGroupsPerWave == 4, "2 or 4 groups per wave");
constexpr int kTiledKC = 4;                             // 32-deep steps per staged chunk (128 deep)
constexpr int kTiledFrags = 2 * kTiledKC;               // 16-deep fragments per row block and chunk
constexpr int kTiledSlot = 1056;                        // bytes per fragment slot (1 KiB + bank padding)
constexpr int kTiledHalfOff = 528;                      // byte offset of reduction half 1 in a slot
constexpr int kTiledBuf = kTiledRowBlocks * kTiledFrags * kTiledSlot;  // bytes per LDS buffer
constexpr int kTiledLoads = 8;                          // staging loads per wave and chunk (4 rows each)
#ifndef AFD_TILED_B_AHEAD
#define AFD_TILED_B_AHEAD (8 / AFD_TILED_GPW)
#endif
constexpr int kTiledBAhead = AFD_TILED_B_AHEAD;         // 32-deep weight steps in flight per wave
constexpr int kXcds = 8;

static_assert(kTiledRowBlocks == kTiledWaves, "each wave stages one 32-row block");
static_assert(kTiledLoads * 4 == 32, "a wave stages 32 rows, 4 per load");

__device__ __forceinline__ bf16x8 tiled_load_b(const bf16x8* p) { return *p; }

template <int N>
struct IntC {
  static constexpr int value = N;
};

#ifndef AFD_TILED_SCHED
#define AFD_TILED_SCHED 1
#endif

#ifndef AFD_TILED_MIN_BLOCKS
#define AFD_TILED_MIN_BLOCKS 1
#endif
constexpr int kTiledMinBlocks = AFD_TILED_MIN_BLOCKS;  // workgroups per CU the registers must allow

template <bool SWIGLU>
__global__ void __launch_bounds__(kTiledThreads, kTiledMinBlocks) gemm_bf16_tiled_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kTiledWaves + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int total = build_item_prefix(g, kTiledRows, kTiledGroups, prefix, scan_tmp);
  const int w = threadIdx.x / kWave;

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
    const int NC = KB / kTiledKC;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    // First group of this wave.  A wave past the last group of a partial column tile
    // recomputes the tile's last groups and stores nothing: the main loop stays free
    // of branches around the MFMAs (such a branch made the compiler copy every
    // accumulator through VGPRs).  Group counts are multiples of 4, so a wave's groups
    // are all valid or all past the end.
    const bool active = it.group + w * kTiledGroupsPerWave < groups;  // wave-uniform
    const int group0 = active ? it.group + w * kTiledGroupsPerWave : groups - kTiledGroupsPerWave;

    // Rows this wave stages: w * 32 + i * 4 + lane / 16 (i = 0..7), clamped into the
    // tile; the lane carries the 16-byte piece lane % 16 of each row's 256-byte chunk.
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const __bf16* abase = static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed);
    const int piece = lane & 15;
    const bf16x8* arow[kTiledLoads];
#pragma unroll
    for (int i = 0; i < kTiledLoads; ++i) {
      int r = w * 32 + i * 4 + (lane >> 4);
      r = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[i] = reinterpret_cast<const bf16x8*>(abase + (size_t)ar * lda) + piece;
    }
    // LDS byte offsets: where this lane's staged piece goes (row block w, fragment
    // piece / 2, reduction half piece % 2; + i * 64 for load i), and where it reads
    // its A operand (fragment slot base + lane position)
    const int wr_off = (w * kTiledFrags + (piece >> 1)) * kTiledSlot + (lane >> 4) * 16 + (piece & 1) * kTiledHalfOff;
    const int rd_off = (lane & 31) * 16 + (lane >> 5) * kTiledHalfOff;

    // weights: 16-byte chunk of (step s, half kh) for block cb at bbase[cb] + s*128 + kh*32
    const __bf16* wbase = it.shared ? static_cast<const __bf16*>(g.w_shared)
                                    : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const bf16x8* bbase[kTiledGroupsPerWave];
#pragma unroll
    for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) {
      const int grp = SWIGLU ? group0 + (cb >> 1) * 2 + ((lane & 31) >> 4) : group0 + cb;
      const int half = SWIGLU ? (cb & 1) : ((lane & 31) >> 4);
      bbase[cb] = reinterpret_cast<const bf16x8*>(wbase) + (size_t)grp * KB * 128 + half * 64 + (lane >> 5) * 16 +
                  (lane & 15);
    }

    f32x16v acc[kTiledRowBlocks][kTiledGroupsPerWave];
#pragma unroll
    for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) acc[rb][cb] = f32x16v{};

    // weight ring: step s lives in slot s % kTiledBAhead ([cb][kh])
    bf16x8 bring[kTiledBAhead][kTiledGroupsPerWave][2];
#pragma unroll
    for (int u = 0; u < kTiledBAhead; ++u)
#pragma unroll
      for (int cb = 0; cb < kTiledGroupsPerWave; ++cb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) bring[u][cb][kh] = tiled_load_b(bbase[cb] + u * 128 + kh * 32);

    // The main loop is instantiated for RB = 1..4 row blocks holding rows, so a tile
    // with few rows does only the MFMAs, LDS reads and activation staging its rows
    // need (waves w >= RB stage nothing; every wave still takes the barriers).  RB is
    // uniform over the workgroup.
    auto main_loop = [&](auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      // A chunk 0 -> LDS buffer 0, chunk 1 (or chunk 0 again) -> staging registers;
      // a chunk is 16 pieces of 16 bytes per row
      bf16x8 stage[kTiledLoads];
      if (w < RB) {
#pragma unroll
        for (int i = 0; i < kTiledLoads; ++i) stage[i] = arow[i][0];
#pragma unroll
        for (int i = 0; i < kTiledLoads; ++i) *reinterpret_cast<bf16x8*>(lds + wr_off + i * 64) = stage[i];
        const int cn = NC > 1 ? 1 : 0;
#pragma unroll
        for (int i = 0; i < kTiledLoads; ++i) stage[i] = arow[i][cn * 16];
      }
      __syncthreads();

      // The reduction runs as 16-deep half-steps (u, kh).  The A fragments of the next
      // half-step are read from LDS while the current half-step's MFMAs run; in the
      // chunk's last half-step the next chunk (already in registers) is written to the
      // other LDS buffer and the barrier is taken before its first fragments are read,
      // so that read is covered by the last MFMAs of this chunk too.
      bf16x8 a[2][kTiledRowBlocks];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a[0][rb] = *reinterpret_cast<const bf16x8*>(lds + rb * kTiledFrags * kTiledSlot + rd_off);

      for (int c = 0; c < NC; ++c) {
        const int buf = (c & 1) * kTiledBuf;
        const int nbuf = kTiledBuf - buf;
#pragma unroll
        for (int hs = 0; hs < kTiledFrags; ++hs) {
          const int u = hs >> 1, kh = hs & 1;
          const int cur = hs & 1, nxt = cur ^ 1;
          if (hs + 1 < kTiledFrags) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[nxt][rb] =
                  *reinterpret_cast<const bf16x8*>(lds + buf + (rb * kTiledFrags + hs + 1) * kTiledSlot + rd_off);
          } else {
            // branch-free chunk boundary: past the last chunk these write, load and read
            // data nobody uses (the loads are clamped to the last chunk)
            if (w < RB) {
#pragma unroll
              for (int i = 0; i < kTiledLoads; ++i)
                *reinterpret_cast<bf16x8*>(lds + nbuf + wr_off + i * 64) = stage[i];
            }
            __syncthreads();
            if (w < RB) {
              const int cn = c + 2 < NC ? c + 2 : NC - 1;
#pragma unroll
              for (int i = 0; i < kTiledLoads; ++i) stage[i] = arow[i][cn * 16];
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[nxt][rb] = *reinterpret_cast<const bf16x8*>(lds + nbuf + rb * kTiledFrags * kTiledSlot + rd_off);
          }
          const int slotb = u % kTiledBAhead;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < kTiledGroupsPerWave; ++cb)
              acc[rb][cb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][rb], bring[slotb][cb][kh], acc[rb][cb], 0, 0, 0);
          if (kh == 1) {
            // refill this ring slot with the step kTiledBAhead ahead (clamped to the last)
            int s = c * kTiledKC + u + kTiledBAhead;
            s = s < KB ? s : KB - 1;
#pragma unroll
            for (int cb = 0; cb < kTiledGroupsPerWave; ++cb)
#pragma unroll
              for (int k2 = 0; k2 < 2; ++k2) bring[slotb][cb][k2] = tiled_load_b(bbase[cb] + s * 128 + k2 * 32);
          }
#if AFD_TILED_SCHED
          // keep the next half-step's LDS reads spread between this half-step's MFMAs
          // (left alone, the scheduler sinks each read to just before its first use)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, kTiledGroupsPerWave, 0);  // one row block's MFMAs
          }
#endif
        }
      }
    };
    // Only an expert's single row tile is shortened: the row tiles of a larger
    // expert stream the same weights at the same time through one XCD's L2, and a
    // shortened last tile running ahead of its siblings measured slower.
    const int seg_rows = it.shared ? g.shared_rows : g.counts[it.seg];
    const int nrb = seg_rows > kTiledRows ? kTiledRowBlocks : (it.nrows + 31) / 32;
    if (nrb >= 4)
      main_loop(IntC<4>{});
    else if (nrb == 3)
      main_loop(IntC<3>{});
    else if (nrb == 2)
      main_loop(IntC<2>{});
    else
      main_loop(IntC<1>{});

    if (active) {
      const int col = lane & 31;
      const int rsub = (lane >> 5) * 4;
      if (SWIGLU) {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < it.nrows) {
              __bf16* o = out + (size_t)(it.row0 + row) * ldo + group0 * 16 + col;
#pragma unroll
              for (int p = 0; p < kTiledGroupsPerWave / 2; ++p)
                o[p * 32] = f32_to_bf16(silu(acc[rb][2 * p][i]) * acc[rb][2 * p + 1][i]);
            }
          }
      } else {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < it.nrows) {
              __bf16* o = out + (size_t)(it.row0 + row) * ldo + group0 * 32 + col;
#pragma unroll
              for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) o[cb * 32] = f32_to_bf16(acc[rb][cb][i]);
            }
          }
      }
    }
    // every LDS read of this item was issued before the barrier of its last half-step,
    // so the next item's first LDS writes need no further barrier
  }
}

template <bool SWIGLU>
static hipError_t launch_tiled(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = 2 * kTiledBuf;  // above the default limit: see configure_gemm_bf16_tiled
  // max_blocks counts compute units; the kernel is built for kTiledMinBlocks
  // resident workgroups on each
  const long long resident = (long long)max_blocks * kTiledMinBlocks;
  long long blocks = max_items < resident ? max_items : resident;
  blocks = blocks < kXcds ? kXcds : blocks / kXcds * kXcds;
  gemm_bf16_tiled_kernel<SWIGLU><<<(unsigned)blocks, kTiledThreads, smem, st>>>(g);
  return hipGetLastError();
}

// Every reduction length here is a multiple of 128 (the layer's dimensions are), so
// whole 128-deep chunks cover it.
// Raise the kernels' dynamic LDS limit on the current device (handle creation).
hipError_t configure_gemm_bf16_tiled() {
  const int smem = 2 * kTiledBuf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_tiled_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_tiled_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  return e;
}

hipError_t launch_gemm_bf16_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                  hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  if (g.K_routed % 128 || (g.shared_rows > 0 && g.K_shared % 128)) return hipErrorInvalidValue;
  return swiglu ? launch_tiled<true>(g, max_items, max_blocks, st) : launch_tiled<false>(g, max_items, max_blocks, st);
}

int tiled_rows() { return kTiledRows; }
int tiled_groups() { return kTiledGroups; }

}  // namespace afd
