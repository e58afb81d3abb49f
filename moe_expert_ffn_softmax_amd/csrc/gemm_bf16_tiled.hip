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
//
// A workgroup's items run as one stream: during an item's last chunks the activation
// staging and the weight ring already load the next item's first chunks and steps,
// so the next item starts without waiting for its first loads (measured: the start-up
// latency of an item was 5-9% of the launch at 128 to 1024 rows per expert).
#include "grouped.h"

namespace afd {

typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int kTiledWaves = 4;
constexpr int kTiledThreads = kTiledWaves * kWave;
constexpr int kTiledRowBlocks = 4;                      // 32-row blocks per tile (one per staging wave)
constexpr int kTiledRows = 32 * kTiledRowBlocks;        // 128
constexpr int kTiledGroupsPerWave = 2;                 // 32-column groups per wave (2 or 4)
constexpr int kTiledGroups = kTiledWaves * kTiledGroupsPerWave;  // per item
static_assert(kTiledGroupsPerWave == 2 || kTiledGroupsPerWave == 4, "2 or 4 groups per wave");
constexpr int kTiledKC = 4;                             // 32-deep steps per staged chunk (128 deep)
constexpr int kTiledFrags = 2 * kTiledKC;               // 16-deep fragments per row block and chunk
constexpr int kTiledSlot = 1056;                        // bytes per fragment slot (1 KiB + bank padding)
constexpr int kTiledHalfOff = 528;                      // byte offset of reduction half 1 in a slot
constexpr int kTiledBuf = kTiledRowBlocks * kTiledFrags * kTiledSlot;  // bytes per LDS buffer
constexpr int kTiledLoads = 8;                          // staging loads per wave and chunk (4 rows each)
constexpr int kTiledBAhead = 8 / kTiledGroupsPerWave;   // 32-deep weight steps in flight per wave
// a ring slot is the step's index within its chunk modulo the ring depth
static_assert(kTiledKC % kTiledBAhead == 0, "the weight ring depth divides the steps of a chunk");
constexpr int kXcds = 8;

static_assert(kTiledRowBlocks == kTiledWaves, "each wave stages one 32-row block");
static_assert(kTiledLoads * 4 == 32, "a wave stages 32 rows, 4 per load");

__device__ __forceinline__ bf16x8 tiled_load_b(const bf16x8* p) { return *p; }

template <int N>
struct IntC {
  static constexpr int value = N;
};

constexpr int kTiledMinBlocks = 1;  // workgroups per CU the registers must allow

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// SiLU with the hardware reciprocal (one rounding more than z / (1 + e^-z)); h is
// rounded to bf16 right after.
__device__ __forceinline__ float silu_rcp(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Addressing of one work item for one wave: the rows it stages and the weight streams
// of its groups.  Item-level values are wave-uniform (scalar registers); per lane
// there are only 32-bit offsets.
struct TiledCtx {
  int seg, shared, row0, nrows;
  int KB, NC;      // 32-deep steps and 128-deep chunks of the reduction
  int active;      // the wave's groups exist (else it recomputes the last ones, stores nothing)
  int group0;      // first group of the wave
  const bf16x8* abase;                    // the A matrix
  uint32_t aoff[kTiledLoads];             // this lane's piece of each staged row (bf16x8 units)
  const bf16x8* wbase;                    // the expert's packed weights
  uint32_t boff[kTiledGroupsPerWave];     // this lane's weight stream of each block (bf16x8 units)
};

template <bool SWIGLU>
__device__ __forceinline__ void tiled_ctx(const GroupedGemm& g, const SegTable& prefix, int item, int w, int lane,
                                          TiledCtx& x) {
  const Item it = decode_item_tiled(g, kTiledRows, kTiledGroups, prefix, item);
  x.seg = uni(it.seg);
  x.shared = uni(it.shared ? 1 : 0);
  x.row0 = uni(it.row0);
  x.nrows = uni(it.nrows);
  const int K = x.shared ? g.K_shared : g.K_routed;
  x.KB = K / 32;
  x.NC = x.KB / kTiledKC;
  const int groups = x.shared ? g.groups_shared : g.groups_routed;
  const int group = uni(it.group);
  // A wave past the last group of a partial column tile recomputes the tile's last
  // groups and stores nothing: the main loop stays free of branches around the MFMAs
  // (such a branch made the compiler copy every accumulator through VGPRs).  Group
  // counts are multiples of 4, so a wave's groups are all valid or all past the end.
  x.active = group + w * kTiledGroupsPerWave < groups;
  x.group0 = x.active ? group + w * kTiledGroupsPerWave : groups - kTiledGroupsPerWave;
  // Rows this wave stages: w * 32 + i * 4 + lane / 16 (i = 0..7), clamped into the
  // tile; the lane carries the 16-byte piece lane % 16 of each row's 256-byte chunk.
  const int lda = x.shared ? g.lda_shared : g.lda_routed;
  x.abase = static_cast<const bf16x8*>(x.shared ? g.a_shared : g.a_routed);
  // The sorted_pair lookups are all issued before the first is used: in a branch per
  // row, each would wait for its load (and every load in flight) before the next one
  // issues.
  int ar[kTiledLoads];
#pragma unroll
  for (int i = 0; i < kTiledLoads; ++i) {
    const int r = w * 32 + i * 4 + (lane >> 4);
    ar[i] = x.row0 + (r < x.nrows ? r : 0);
  }
  if (!x.shared && g.gather_routed) {
#pragma unroll
    for (int i = 0; i < kTiledLoads; ++i) ar[i] = g.sorted_pair[ar[i]];
#pragma unroll
    for (int i = 0; i < kTiledLoads; ++i) ar[i] /= g.k;
  }
#pragma unroll
  for (int i = 0; i < kTiledLoads; ++i) x.aoff[i] = (uint32_t)ar[i] * (uint32_t)(lda / 8) + (uint32_t)(lane & 15);
  // weights: 16-byte chunk of (step s, half kh) of block cb at boff[cb] + s*128 + kh*32
  x.wbase = x.shared ? static_cast<const bf16x8*>(g.w_shared)
                     : static_cast<const bf16x8*>(g.w_routed) + (size_t)x.seg * (g.w_expert_elems / 8);
#pragma unroll
  for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) {
    const int grp = SWIGLU ? x.group0 + (cb >> 1) * 2 + ((lane & 31) >> 4) : x.group0 + cb;
    const int half = SWIGLU ? (cb & 1) : ((lane & 31) >> 4);
    x.boff[cb] = (uint32_t)grp * (uint32_t)(x.KB * 128) + half * 64 + (lane >> 5) * 16 + (lane & 15);
  }
}

// The work items of a workgroup run as one stream: during an item's last chunks the
// staging loads and the weight ring already fetch the next item's first chunk and
// steps (when both items have at least two chunks), so the next item starts without
// the latency of its first loads.  The next item's addresses (which need its rows'
// sorted_pair entries) are computed at the start of the current one.
template <bool SWIGLU>
__global__ void __launch_bounds__(kTiledThreads, kTiledMinBlocks) gemm_bf16_tiled_kernel(GroupedGemm g) {
  __shared__ SegTable prefix;
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
  int item = begin + slot;
  if (item >= end) return;  // uniform over the workgroup

  const int lane = lane_id();
  const int piece = lane & 15;
  // LDS byte offsets: where this lane's staged piece goes (row block w, fragment
  // piece / 2, reduction half piece % 2; + i * 64 for load i), and where it reads
  // its A operand (fragment slot base + lane position)
  const int wr_off = (w * kTiledFrags + (piece >> 1)) * kTiledSlot + (lane >> 4) * 16 + (piece & 1) * kTiledHalfOff;
  const int rd_off = (lane & 31) * 16 + (lane >> 5) * kTiledHalfOff;

  TiledCtx cur;
  tiled_ctx<SWIGLU>(g, prefix, item, w, lane, cur);

  f32x16v acc[kTiledRowBlocks][kTiledGroupsPerWave];
#pragma unroll
  for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
    for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) acc[rb][cb] = f32x16v{};
  // weight ring: step s lives in slot s % kTiledBAhead ([cb][kh])
  bf16x8 bring[kTiledBAhead][kTiledGroupsPerWave][2];
  bf16x8 stage[kTiledLoads];  // the staged chunk after the one in LDS
  int base = 0;               // LDS buffer of the current item's chunk 0
  bool primed = false;        // ring, LDS chunk 0 and stage already hold this item's data

  for (;;) {
    const int item_n = item + slots;
    const bool has_next = item_n < end;
    TiledCtx nxt;
    if (has_next)
      tiled_ctx<SWIGLU>(g, prefix, item_n, w, lane, nxt);
    else
      nxt = cur;
    // chaining needs two chunks on both sides (the staging runs two chunks ahead) and
    // ring slots that line up across the item boundary
    const bool chain = has_next && cur.NC >= 2 && nxt.NC >= 2 && cur.KB % kTiledBAhead == 0;

    if (!primed) {
#pragma unroll
      for (int u = 0; u < kTiledBAhead; ++u)
#pragma unroll
        for (int cb = 0; cb < kTiledGroupsPerWave; ++cb)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
            bring[u][cb][kh] = tiled_load_b(cur.wbase + cur.boff[cb] + (u < cur.KB ? u : cur.KB - 1) * 128 + kh * 32);
      // chunk 0 -> LDS buffer `base`, chunk 1 (or chunk 0 again) -> staging registers;
      // a chunk is 16 pieces of 16 bytes per row
#pragma unroll
      for (int i = 0; i < kTiledLoads; ++i) stage[i] = cur.abase[cur.aoff[i]];
#pragma unroll
      for (int i = 0; i < kTiledLoads; ++i)
        *reinterpret_cast<bf16x8*>(lds + base * kTiledBuf + wr_off + i * 64) = stage[i];
      const int cn = cur.NC > 1 ? 1 : 0;
#pragma unroll
      for (int i = 0; i < kTiledLoads; ++i) stage[i] = cur.abase[cur.aoff[i] + cn * 16];
      __syncthreads();
    }

    // The chunk loop runs inside a generic lambda over the row-block count (always
    // all four here): written inline, the compiler schedules it worse (measured 6%
    // slower at 1024 rows per expert).
    auto main_loop = [&](auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      const int NC = cur.NC, KB = cur.KB;
      // The reduction runs as 16-deep half-steps (u, kh).  The A fragments of the next
      // half-step are read from LDS while the current half-step's MFMAs run; in the
      // chunk's last half-step the next chunk (already in registers) is written to the
      // other LDS buffer and the barrier is taken before its first fragments are read,
      // so that read is covered by the last MFMAs of this chunk too.
      bf16x8 a[2][kTiledRowBlocks];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a[0][rb] = *reinterpret_cast<const bf16x8*>(lds + base * kTiledBuf + rb * kTiledFrags * kTiledSlot + rd_off);

      for (int c = 0; c < NC; ++c) {
        const int buf = ((base + c) & 1) * kTiledBuf;
        const int nbuf = kTiledBuf - buf;
#pragma unroll
        for (int hs = 0; hs < kTiledFrags; ++hs) {
          const int u = hs >> 1, kh = hs & 1;
          const int cur_a = hs & 1, nxt_a = cur_a ^ 1;
          if (hs + 1 < kTiledFrags) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[nxt_a][rb] =
                  *reinterpret_cast<const bf16x8*>(lds + buf + (rb * kTiledFrags + hs + 1) * kTiledSlot + rd_off);
          } else {
            // chunk boundary: the staged chunk goes to the other buffer, then the chunk
            // two ahead is staged: this item's, the next item's first ones when
            // chaining, else a clamped load nobody uses
#pragma unroll
            for (int i = 0; i < kTiledLoads; ++i)
              *reinterpret_cast<bf16x8*>(lds + nbuf + wr_off + i * 64) = stage[i];
            __syncthreads();
            const int c2 = c + 2;
            const bool own = c2 < NC;
            const bool take_next = !own && chain;  // uniform
            const int cc = own ? c2 : take_next ? c2 - NC : NC - 1;
            const bf16x8* ab = take_next ? nxt.abase : cur.abase;
#pragma unroll
            for (int i = 0; i < kTiledLoads; ++i)
              stage[i] = ab[(take_next ? nxt.aoff[i] : cur.aoff[i]) + cc * 16];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              a[nxt_a][rb] = *reinterpret_cast<const bf16x8*>(lds + nbuf + rb * kTiledFrags * kTiledSlot + rd_off);
          }
          const int slotb = u % kTiledBAhead;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < kTiledGroupsPerWave; ++cb)
              acc[rb][cb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur_a][rb], bring[slotb][cb][kh], acc[rb][cb], 0, 0, 0);
          if (kh == 1) {
            // refill this ring slot with the step kTiledBAhead ahead: this item's, the
            // next item's first steps when chaining, else the last step again
            const int s = c * kTiledKC + u + kTiledBAhead;
            const bool own = s < KB;
            const bool take_next = !own && chain;  // uniform
            const int ss = own ? s : take_next ? s - KB : KB - 1;
            const bf16x8* wb = take_next ? nxt.wbase : cur.wbase;
#pragma unroll
            for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) {
              const bf16x8* bp = wb + (take_next ? nxt.boff[cb] : cur.boff[cb]) + ss * 128;
#pragma unroll
              for (int k2 = 0; k2 < 2; ++k2) bring[slotb][cb][k2] = tiled_load_b(bp + k2 * 32);
            }
          }
          // keep the next half-step's LDS reads spread between this half-step's MFMAs
          // (left alone, the scheduler sinks each read to just before its first use)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, kTiledGroupsPerWave, 0);  // one row block's MFMAs
          }
        }
      }
    };
    main_loop(IntC<4>{});

    if (cur.active) {
      const int col = lane & 31;
      const int rsub = (lane >> 5) * 4;
      __bf16* out = static_cast<__bf16*>(cur.shared ? g.out_shared : g.out_routed);
      const int ldo = cur.shared ? g.ldo_shared : g.ldo_routed;
      if (SWIGLU) {
#pragma unroll
        for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < cur.nrows) {
              __bf16* o = out + (size_t)(cur.row0 + row) * ldo + cur.group0 * 16 + col;
#pragma unroll
              for (int p = 0; p < kTiledGroupsPerWave / 2; ++p)
                o[p * 32] = f32_to_bf16(silu_rcp(acc[rb][2 * p][i]) * acc[rb][2 * p + 1][i]);
            }
          }
      } else {
#pragma unroll
        for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rb * 32 + (i / 4) * 8 + rsub + (i % 4);
            if (row < cur.nrows) {
              __bf16* o = out + (size_t)(cur.row0 + row) * ldo + cur.group0 * 32 + col;
#pragma unroll
              for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) o[cb * 32] = f32_to_bf16(acc[rb][cb][i]);
            }
          }
      }
    }
    if (!has_next) break;
#pragma unroll
    for (int rb = 0; rb < kTiledRowBlocks; ++rb)
#pragma unroll
      for (int cb = 0; cb < kTiledGroupsPerWave; ++cb) acc[rb][cb] = f32x16v{};
    // the last chunk boundary wrote the next item's chunk 0 (or, unchained, a chunk
    // nobody reads) to buffer (base + NC) % 2 and took a barrier after every read of
    // this item's data
    base = (base + cur.NC) & 1;
    primed = chain;
    cur = nxt;
    item = item_n;
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
