// Grouped expert GEMMs with fp8 (OCP e4m3) operands and fp32 block scales, large-tile
// form: the fp8 counterpart of the bf16 128-row tiled kernel, for layers whose experts
// receive many rows (the DeepSeek-V3-like layer of an FFN instance aggregating
// attention batches; FP8/BF16 mixed precision: the omica.com.cn AFD article, §3.3).
//
// A workgroup of 8 waves (two per SIMD) computes a 128-token tile of one expert times
// 8 32-column groups; wave w owns group w for all 128 tokens.  The matrix-core
// instruction is v_mfma_f32_16x16x128_f8f6f4 (the scaled builtin with zero scale
// operands, which the compiler emits as the unscaled instruction): one instruction
// covers one 128-deep scale block of a 16 x 16 output block, and its fp32 partial
// product is added to the accumulator times s_act[token][kb] * s_w[kb][nb].
//
// Operand roles.  The weights are the instruction's first operand and the tokens its
// second, so the 16 x 16 result is (weight column) x (token): lane l holds columns
// (l / 16) * 4 .. + 3 of token l % 16.  Each lane then needs one activation scale per
// token block and scale block, and the weight scale is uniform over a 16-column
// block: rescaling a partial product is one multiply and four FMAs.  Lane l supplies
// column (or token) l % 16 at reduction offsets (l / 16) * 32 .. + 31 of the 128-deep
// block; the packed weight layout (see gemm_fp8.hip) keeps a fragment in one 2 KiB
// run whose two halves each give every lane 16 of its bytes, so each of a fragment's
// two loads reads 1 KiB contiguously.
//
// Activation staging.  A 256-deep chunk (two scale blocks) of the 128 gathered token
// rows is loaded as 4 rows x 256 contiguous bytes per instruction (lane l: row l / 16,
// 16-byte piece l % 16) and written to LDS in operand order: token block b (16 rows)
// has 16 slots of 272 bytes, slot q holding piece q of its 16 rows at (row % 16) * 16.
// Piece q of a chunk is (scale block q / 8, reduction group (q % 8) / 2, 16-byte half
// q % 2) of the operand.  The 16 lanes writing one row hit 16 different bank groups;
// a 16-lane quarter of an operand read is one slot, contiguous.  Double-buffered; the
// next chunk is loaded into registers while the current one is multiplied.  Each wave
// stages one 16-row block.
//
// The chunk's token scales and the weight scales of its two blocks are staged through
// LDS beside the activations (one scale per lane per chunk), so inside a block the only
// memory waits are for the weight ring.  Every staging load is issued unconditionally
// and its value is first used at the LDS write a chunk later: a load under a divergent
// branch, or one whose value is used at once, makes the compiler wait for every load
// in flight, the weight ring's included.
//
// Schedule of a block.  Rescaling costs one multiply and four FMAs per MFMA, about
// half the MFMA time; with two waves per SIMD one wave's rescaling overlaps the other
// wave's MFMAs, and within a wave the instruction order interleaves them.  Each step
// rb of a block issues block rb's first MFMA, then the LDS reads of token block rb + 1's
// operand, then the rescaling of block rb - 1's products (kept in a second register
// set) around block rb's second MFMA.  The compiler would
// otherwise gather the pure arithmetic of the whole unrolled block in one place, so
// empty asm statements that consume a step's products and accumulators keep each step
// between scheduling barriers.
//
// For the gate/up projection the epilogue can write h already quantised (e4m3 codes
// and per-token per-128 scales; see below) instead of fp32 h.
//
// Items as in the bf16 tiled kernel; the XCD ranges carry equal costs (f8_xcd_range).
// A workgroup takes its items as runs: consecutive items (of its strided sequence)
// with the same count of 16-row blocks share one body specialised on that count.  In
// the down projection the items of a run are chained: an item's last chunk loads the
// next item's first chunks and weight blocks where it would otherwise reload its own,
// so the next item starts without waiting for memory (see the kernel).  The gate/up
// projection, whose items are 3.5x longer, measured no faster chained and runs each
// item on its own.
#include "grouped.h"

namespace afd {

constexpr int kF8Waves = 8;                     // two per SIMD
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8RowBlocks = 8;                 // 16-token blocks per tile
constexpr int kF8Rows = 16 * kF8RowBlocks;      // 128
constexpr int kF8Groups = 8;                    // 32-column groups per tile (one h quantisation group)
constexpr int kF8GroupsPerWave = kF8Groups / kF8Waves;  // 32-column groups per wave
constexpr int kF8CB = 2 * kF8GroupsPerWave;     // 16-column blocks per wave
constexpr int kF8Slot = 272;                    // bytes per staging slot (16 rows x 16 B + padding)
constexpr int kF8A = kF8RowBlocks * 16 * kF8Slot;  // activation bytes per buffer
constexpr int kF8WScales = 2 * kF8Waves * kF8CB;  // weight scales per chunk (2 blocks)
// + the chunk's token and weight scales, and one 16-byte word that the threads with no
// scale to stage write to
constexpr int kF8Buf = kF8A + 2 * kF8Rows * 4 + kF8WScales * 4 + 16;
constexpr int kF8Dummy = kF8A + 2 * kF8Rows * 4 + kF8WScales * 4;  // byte offset of that word
constexpr int kF8StageRows = kF8Rows / kF8Waves;  // rows each wave stages per chunk
constexpr int kF8Loads = kF8StageRows / 4;      // staging loads per thread per chunk (4 rows each)
// Each wave stages its rows' token scales of a chunk (2 blocks) in lanes 0-31 and the
// chunk's weight scales in lanes 32-63 (written by wave 0 only): one load per lane.
static_assert(2 * kF8StageRows + kF8WScales == kWave, "one scale per lane per chunk");
// Weight blocks in flight per wave: one chunk's two scale blocks (ring slot = the
// block's index in its chunk).  The staging registers hold one chunk.
constexpr int kF8BAhead = 2;
constexpr int kF8LdsAhead = 1;                  // token blocks of operands read from LDS ahead
constexpr int kF8Xcds = 8;

__device__ __forceinline__ f32x4 f8_mfma(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // scale operands 0: the compiler emits the unscaled v_mfma_f32_16x16x128_f8f6f4
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Global-memory views of pointers rebuilt from scalar registers (without them the
// compiler emits flat loads, which also count against the LDS wait counter).
typedef const __attribute__((address_space(1))) uint8_t gu8;
typedef const __attribute__((address_space(1))) float gf32;
typedef const __attribute__((address_space(1))) bf16x8 gbf16x8;
typedef const __attribute__((address_space(1))) i32x4 gi32x4;
// A lane's 32 weight bytes of a packed fragment: 16 at p, 16 at p + 1 KiB.
__device__ __forceinline__ i32x8 f8_load32g(gu8* p) {
  gi32x4* q = reinterpret_cast<gi32x4*>(p);
  const i32x4 lo = q[0], hi = q[64];
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

constexpr int kF8MinBlocks = 1;  // workgroups per CU the registers must allow

// SiLU with the hardware reciprocal (one rounding more than z / (1 + e^-z)); h is
// quantised to e4m3 right after, whose step is 2^-3 of the value.
__device__ __forceinline__ float silu_rcp(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// A pointer held in scalar registers (the value must be the same in every lane).
template <typename T>
__device__ __forceinline__ T* f8_uniform(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}

// What an item's loads read: the rows it stages (gathered through sorted_pair for
// routed gate/up rows), its token and weight block scales, and the wave's weight
// fragments.  Bases are wave-uniform (scalar registers) and the per-lane parts 32-bit
// byte offsets, so that a load is one instruction on a scalar base and a vector offset
// (no 64-bit address arithmetic per load).
struct F8Src {
  const uint8_t* abase;         // activation rows of the item's segment (uniform)
  unsigned aoff[kF8Loads];      // staged row w*kF8StageRows + i*4 + lane/16: byte offset from abase
  const float* sp;              // the scale this lane stages, at block 0 (token scales for lanes
                                //   < 32, weight scales for lanes >= 32)
  int sstep;                    // floats between consecutive blocks' scales of this lane
  const uint8_t* Bu;            // the wave's weight fragments (uniform; lane l reads at l * 16)
  unsigned gs;                  // bytes per 32-column group of weights (uniform)
  int K, KB;                    // reduction length, 128-deep blocks (uniform)
};

// Issue the sorted_pair lookups of an item's staged rows and of this thread's token-scale
// row.  Branch-free: rows that are not gathered read counts[0], which f8_source ignores
// (a load under a wave-uniform branch makes the compiler's later waits conservative).
__device__ __forceinline__ void f8_lookup(const GroupedGemm& g, const Item& it, int w, int lane,
                                          int (&lk)[kF8Loads + 1]) {
  const bool gather = !it.shared && g.gather_routed;
  const int32_t* src = gather ? g.sorted_pair : g.counts;
#pragma unroll
  for (int i = 0; i < kF8Loads; ++i) {
    const int r = w * kF8StageRows + i * 4 + (lane >> 4);
    lk[i] = src[gather ? it.row0 + (r < it.nrows ? r : 0) : 0];
  }
  const int t = w * kF8StageRows + (lane & (kF8StageRows - 1));
  lk[kF8Loads] = src[gather ? it.row0 + (t < it.nrows ? t : 0) : 0];
}

// An item's sources, from its lookups (the first use of their values).
template <bool SWIGLU>
__device__ __forceinline__ void f8_source(const GroupedGemm& g, const Item& it, int w, int lane,
                                          const int (&lk)[kF8Loads + 1], F8Src& s) {
  const bool gather = !it.shared && g.gather_routed;
  s.K = it.shared ? g.K_shared : g.K_routed;
  s.KB = s.K / 128;
  const int groups = it.shared ? g.groups_shared : g.groups_routed;
  const int N = groups * 32;
  const int NB = N / 128;
  const unsigned lda = (unsigned)(it.shared ? g.lda_shared : g.lda_routed);
  s.abase = f8_uniform(static_cast<const uint8_t*>(it.shared ? g.a_shared : g.a_routed));
#pragma unroll
  for (int i = 0; i < kF8Loads; ++i) {
    const int r = w * kF8StageRows + i * 4 + (lane >> 4);
    const int row = it.row0 + (r < it.nrows ? r : 0);
    s.aoff[i] = (unsigned)(gather ? lk[i] / g.k : row) * lda;
  }
  // a wave past the last group of a partial column tile recomputes the tile's last two
  // groups and stores nothing (group counts are multiples of 4)
  const int group0 = it.group + w * kF8GroupsPerWave < groups ? it.group + w * kF8GroupsPerWave
                                                               : groups - kF8GroupsPerWave;
  const uint8_t* wbase = it.shared ? static_cast<const uint8_t*>(g.w_shared)
                                   : static_cast<const uint8_t*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
  s.gs = (unsigned)s.KB * 4096;
  // 16-column block cb = (group group0 + cb / 2, half cb % 2): 2 KiB per scale block
  s.Bu = f8_uniform(wbase + (size_t)group0 * s.gs);
  const float* ws = it.shared ? g.s_shared : g.s_routed + (size_t)it.seg * g.s_expert_elems;
  if (lane < 2 * kF8StageRows) {
    const int t = w * kF8StageRows + (lane & (kF8StageRows - 1));
    const int row = it.row0 + (t < it.nrows ? t : 0);
    s.sp = (it.shared ? g.as_shared : g.as_routed) + (size_t)(gather ? lk[kF8Loads] / g.k : row) * s.KB;
    s.sstep = 1;
  } else {
    const int t = lane % (kF8WScales / 2);
    const int w2 = t / kF8CB, cb = t % kF8CB;
    const int g0 = it.group + w2 * kF8GroupsPerWave < groups ? it.group + w2 * kF8GroupsPerWave
                                                             : groups - kF8GroupsPerWave;
    const int j = g0 + (cb >> 1), half = cb & 1;
    s.sp = ws + (SWIGLU ? half * (N / 2) + j * 16 : j * 32 + half * 16) / 128;
    s.sstep = NB;
  }
}

template <int N>
struct F8Blocks {
  static constexpr int value = N;
};

// Item epilogue: h (gate/up; quantised to e4m3 when the layer asks for it) or O (down)
// of the item's rows from the accumulators of its NRB 16-row blocks.
template <bool SWIGLU, int NRB>
__device__ __forceinline__ void f8_epilogue(const GroupedGemm& g, const Item& it, int w, int lane,
                                            const f32x4 (&acc)[NRB][kF8CB], float (*qamax)[kF8Rows]) {
  const int groups = it.shared ? g.groups_shared : g.groups_routed;
  const bool active = it.group + w * kF8GroupsPerWave < groups;  // wave-uniform
  const int group0 = active ? it.group + w * kF8GroupsPerWave : groups - kF8GroupsPerWave;
  const int tok = lane & 15;
  const int n0 = (lane >> 4) * 4;
  float* qscale = it.shared ? g.outs_shared : g.outs_routed;
  if (SWIGLU && qscale) {
    // h quantised in place of the separate pass: the tile's 8 groups are exactly one
    // 128-channel quantisation group of each of its tokens (gate/up column tiles are
    // whole, as 2M/32 is a multiple of 8).  Per token: amax over the 4 lanes of each
    // wave holding it, then over the 8 waves through LDS; scale = amax / 448 (1 for an
    // all-zero group); codes = e4m3(v * (1 / scale)) with the reciprocal rounded once
    // per token group, one rounding more than the quantisation kernel's e4m3(v /
    // scale), and SiLU through the hardware reciprocal: h is internal to the layer, and
    // its codes may differ from the streaming path's by one step.
    f32x4 hv[NRB][kF8GroupsPerWave];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < kF8GroupsPerWave; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[rb][j][i] = silu_rcp(acc[rb][2 * j][i]) * acc[rb][2 * j + 1][i];
          m = fmaxf(m, fabsf(hv[rb][j][i]));
        }
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      if (lane < 16) qamax[w][rb * 16 + tok] = m;
    }
    __syncthreads();
    uint8_t* q = static_cast<uint8_t*>(it.shared ? g.out_shared : g.out_routed);
    const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
    const int qgroups = ldo / 128;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int t = rb * 16 + tok;
      float amax = qamax[0][t];
#pragma unroll
      for (int v = 1; v < kF8Waves; ++v) amax = fmaxf(amax, qamax[v][t]);
      const float sc = amax > 0.f ? amax / 448.f : 1.f;
      const float inv = 1.f / sc;  // one division per token group; codes = e4m3(v * (1 / scale))
      if (t < it.nrows) {
        const size_t row = (size_t)(it.row0 + t);
#pragma unroll
        for (int j = 0; j < kF8GroupsPerWave; ++j)
          *reinterpret_cast<uint32_t*>(q + row * ldo + (group0 + j) * 16 + n0) =
              e4m3_pack4(hv[rb][j][0] * inv, hv[rb][j][1] * inv, hv[rb][j][2] * inv, hv[rb][j][3] * inv);
        if (w == 0 && lane < 16) qscale[row * qgroups + it.group / 8] = sc;
      }
    }
    // the next item's first writes to qamax follow its first chunk's barrier
  } else if (active) {
    const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int t = rb * 16 + tok;
      if (t >= it.nrows) continue;
#pragma unroll
      for (int j = 0; j < kF8GroupsPerWave; ++j) {
        if (SWIGLU) {
          float* o = static_cast<float*>(it.shared ? g.out_shared : g.out_routed) + (size_t)(it.row0 + t) * ldo;
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu(acc[rb][2 * j][i]) * acc[rb][2 * j + 1][i];
          *reinterpret_cast<f32x4*>(o + (group0 + j) * 16 + n0) = v;
        } else {
          // bf16 output rows for the combine: 4 consecutive channels, one 8-byte store
          __bf16* orow = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed) +
                         (size_t)(it.row0 + t) * ldo;
#pragma unroll
          for (int hlf = 0; hlf < 2; ++hlf) {
            const f32x4 v = acc[rb][2 * j + hlf];
            uint2 pk;
            pk.x = (uint32_t)bf16_bits(f32_to_bf16(v[0])) | ((uint32_t)bf16_bits(f32_to_bf16(v[1])) << 16);
            pk.y = (uint32_t)bf16_bits(f32_to_bf16(v[2])) | ((uint32_t)bf16_bits(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(orow + (group0 + j) * 32 + hlf * 16 + n0) = pk;
          }
        }
      }
    }
  }
}

// 16-row blocks an item of `nrows` rows is computed with (its block count, rounded up
// to 4 for 3 blocks and to 2 below that: fewer specialisations of the item body).
__device__ __forceinline__ int f8_item_blocks(int nrows) {
  const int nb = (nrows + 15) / 16;
  return nb >= 5 ? nb : (nb >= 3 ? 4 : 2);
}

// Cost of an item in units of one 16-row block's matrix-core and rescale work: that
// work is proportional to the item's block count, while its weight stream is the same
// for every item.  Measured at the DeepSeek-V3-like layer (ablations of the kernel:
// with and without its loads) the stream weighs about as much as 3 blocks.
constexpr int kF8ItemFixedCost = 3;

// This XCD's range [begin, end) of the launch's items, the 8 ranges carrying equal
// costs rather than equal item counts.  Items differ in cost by their block count, and
// segments are ordered (the shared expert, whose tiles are all full, comes last), so
// equal counts left the last XCD ~10% more work than the mean at that layer.  Within
// a segment all items cost about the same (row counts differ by at most one), so a
// boundary inside a segment is placed by the segment's mean item cost.  costp needs
// kMaxSegments + 1 ints of LDS.  Contains __syncthreads().
__device__ __forceinline__ void f8_xcd_range(const GroupedGemm& g, const SegTable& t, int* costp, int* scan_tmp,
                                             int xcd, int& begin, int& end) {
  const int S = g.E + (g.shared_rows > 0 ? 1 : 0);
  int carry = 0;
  for (int s0 = 0; s0 < S; s0 += blockDim.x) {
    const int s = s0 + threadIdx.x;
    int c = 0;
    if (s < S && t.rows[s] > 0) {
      const int rows = t.rows[s];
      const int rt = (rows + kF8Rows - 1) / kF8Rows;
      const int base = rows / rt, extra = rows - base * rt;  // the row split of decode_item_tiled
      const int groups = s >= g.E ? g.groups_shared : g.groups_routed;
      const int nct = (groups + kF8Groups - 1) / kF8Groups;
      c = nct * (extra * (f8_item_blocks(base + 1) + kF8ItemFixedCost) +
                 (rt - extra) * (f8_item_blocks(base) + kF8ItemFixedCost));
    }
    int tot = 0;
    const int ex = block_exclusive_scan(c, scan_tmp, &tot);
    if (s < S) costp[s] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) costp[S] = carry;
  __syncthreads();
  const long long total_cost = carry;
  // first item whose cost prefix reaches C (by the segment's mean item cost)
  auto item_at = [&](long long C) {
    int lo = 0, hi = S;  // largest lo < S with costp[lo] <= C
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (costp[mid] <= C)
        lo = mid;
      else
        hi = mid;
    }
    const int items = t.prefix[lo + 1] - t.prefix[lo];
    const long long cs = costp[lo + 1] - costp[lo];
    long long local = cs > 0 ? (C - costp[lo]) * items / cs : 0;
    local = local < items ? local : items;
    return t.prefix[lo] + (int)local;
  };
  begin = xcd == 0 ? 0 : item_at(total_cost * xcd / kF8Xcds);
  end = xcd == kF8Xcds - 1 ? t.prefix[S] : item_at(total_cost * (xcd + 1) / kF8Xcds);
}

// The workgroup's items, in runs of equal 16-row block counts (see the item loop).
// CHAIN (down projection with reductions above 256: at least two chunks per item)
// chains the items of a run; without it every item loads its own first chunk and
// weight blocks.
template <bool SWIGLU, bool CHAIN>
__global__ void __launch_bounds__(kF8Threads, kF8MinBlocks) gemm_fp8_tiled_kernel(GroupedGemm g) {
  __shared__ SegTable prefix;
  __shared__ int scan_tmp[kF8Waves + 1];
  __shared__ float qamax[kF8Waves][kF8Rows];  // per-wave token amax of the quantising epilogue
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  __shared__ int costp[kMaxSegments + 1];
  build_item_prefix(g, kF8Rows, kF8Groups, prefix, scan_tmp);
  // wave index, made visibly uniform so that per-wave values (group, scale indices,
  // weight bases) live in scalar registers and use scalar loads
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const int xcd = blockIdx.x % kF8Xcds;
  const int slot = blockIdx.x / kF8Xcds;
  const int slots = gridDim.x / kF8Xcds;
  int begin, end;
  f8_xcd_range(g, prefix, costp, scan_tmp, xcd, begin, end);
  int item = begin + slot;
  if (item >= end) return;  // workgroup-uniform

  const int lane = lane_id();
  const int piece = lane & 15;
  // LDS: write slot of staging load i (token block w, slot = piece, row in block
  // (i % 4) * 4 + lane / 16)
  const int wr_off = ((w * (kF8StageRows / 16)) * 16 + piece) * kF8Slot + (lane >> 4) * 16;
  // read: slot (lane / 16) * 2 (+1 for the upper 16 bytes) of the scale block's 8
  const int rd_off = ((lane >> 4) * 2) * kF8Slot + (lane & 15) * 16;
  // Scales staged with the activations (one per lane per chunk): lane l < 32 stages
  // the value of block l / 16 of the chunk for the wave's row l % 16; lane 32 + u
  // stages, for block u / 16 of the chunk, the scale of wave (u % 16) / kF8CB's
  // 16-column block u % kF8CB (wave 0 writes them, the other waves' copies go to the
  // dummy word).  Loads and LDS writes of the staging are branch-free: a load under a
  // divergent branch whose value is used a chunk later makes the compiler wait, at
  // the use, for every load in flight, the weight ring's included.
  const bool sc_tok = lane < 2 * kF8StageRows;
  const int sc_blk = sc_tok ? lane / kF8StageRows : (lane - 2 * kF8StageRows) / (kF8WScales / 2);
  const int sc_off = sc_tok ? kF8A + (sc_blk * kF8Rows + w * kF8StageRows + (lane % kF8StageRows)) * 4
                            : (w == 0 ? kF8A + (2 * kF8Rows + lane - 2 * kF8StageRows) * 4 : kF8Dummy);

  // The staging registers hold a chunk between its loads and its LDS write.  Rows of
  // token blocks past an item's row count are loaded (reading its first row) and
  // written like the others, and never read.  sstage holds the lane's loaded scale and
  // slive whether its block is inside K (a block past the end of K, odd K / 128, gets
  // weight scale 0): the zeroing is applied when the value is written to LDS, so that
  // no instruction needs the loaded value before the write.
  bf16x8 stage[kF8Loads];
  float sstage;
  bool slive;
  // chunk c of source s's item (clamped to its last chunk; never consumed past it)
  auto load_stage = [&](const F8Src& s, int c) __attribute__((always_inline)) {
    const int nc = (s.KB + 1) / 2;
    c = c < nc ? c : nc - 1;
    // this lane's piece of the chunk (past the end of K: the block before, which gets
    // weight scale 0)
    const unsigned o = c * 256 + piece * 16 < s.K ? piece * 16 : piece * 16 - 128;
    const uint8_t* ab = s.abase + c * 256;
#pragma unroll
    for (int i = 0; i < kF8Loads; ++i) stage[i] = *reinterpret_cast<gbf16x8*>((gu8*)ab + (s.aoff[i] + o));
    const int kb = 2 * c + sc_blk;
    const int kbc = kb < s.KB ? kb : s.KB - 1;
    sstage = ((gf32*)s.sp)[(unsigned)__umul24(kbc, s.sstep)];
    slive = sc_tok || kb < s.KB;
  };
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kF8Loads; ++i)
      *reinterpret_cast<bf16x8*>(lds + buf + wr_off + (i >> 2) * 16 * kF8Slot + (i & 3) * 64) = stage[i];
    *reinterpret_cast<float*>(lds + buf + sc_off) = slive ? sstage : 0.f;
  };
  // weight ring: slot r holds block b of source s's item (clamped to its last block)
  i32x8 bring[kF8BAhead][kF8CB];
  auto load_ring = [&](const int r, const F8Src& s, int b) __attribute__((always_inline)) {
    b = b < s.KB ? b : s.KB - 1;
#pragma unroll
    for (int cb = 0; cb < kF8CB; ++cb)
      bring[r][cb] = f8_load32g((gu8*)s.Bu + ((cb >> 1) * s.gs + (b * 2 + (cb & 1)) * 2048) + (unsigned)(lane * 16));
  };

  // One 128-deep scale block of NRB 16-row blocks: h is the block within the chunk, r
  // its weight-ring slot, buf its LDS buffer.
  auto block = [&](auto nrb, auto& acc, const int h, const int r, const int buf) __attribute__((always_inline)) {
    constexpr int NRB = decltype(nrb)::value;
    const float* swl = reinterpret_cast<const float*>(lds + buf + kF8A) + 2 * kF8Rows + h * (kF8WScales / 2) + w * kF8CB;
    float wsc[kF8CB];
#pragma unroll
    for (int cb = 0; cb < kF8CB; ++cb) wsc[cb] = swl[cb];
    const float* sbuf = reinterpret_cast<const float*>(lds + buf + kF8A) + h * kF8Rows + (lane & 15);
    // Software pipeline over token blocks: block rb + D's operand is read from LDS
    // (D = kF8LdsAhead) and block rb - 1's products are rescaled while block rb's MFMAs
    // run.  The products alternate between two register sets; operands rotate over
    // D + 1 slots and token scales over D + 2, as step rb reads block rb + D's while
    // block rb - 1's is in use.
    constexpr int D = kF8LdsAhead;
    f32x4 p[2][kF8CB];
    i32x8 av[D + 1];
    float sa[D + 2];
    auto rd = [&](const int rb) __attribute__((always_inline)) {
      const unsigned char* ap = lds + buf + (rb * 16 + h * 8) * kF8Slot + rd_off;
      const i32x4 l4 = *reinterpret_cast<const i32x4*>(ap);
      const i32x4 h4 = *reinterpret_cast<const i32x4*>(ap + kF8Slot);
      av[rb % (D + 1)] = i32x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
      sa[rb % (D + 2)] = sbuf[rb * 16];
    };
    auto fm = [&](const int rb) __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < kF8CB; ++cb) {
        const float sc = sa[rb % (D + 2)] * wsc[cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(p[rb & 1][cb][i], sc, acc[rb][cb][i]);
      }
    };
#pragma unroll
    for (int rb = 0; rb < D; ++rb) rd(rb);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      __builtin_amdgcn_sched_barrier(0);
      if (rb + D < NRB) rd(rb + D);
      f32x4* pc = p[rb & 1];
#pragma unroll
      for (int cb = 0; cb < kF8CB; ++cb) pc[cb] = f8_mfma(bring[r][cb], av[rb % (D + 1)]);
      if (rb > 0) fm(rb - 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (rb + D < NRB) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      if (rb > 0) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (rb > 0) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      // keep this step's MFMAs and the previous step's rescaling inside the step
#pragma unroll
      for (int cb = 0; cb < kF8CB; ++cb) asm volatile("" ::"v"(pc[cb]));
      if (rb > 0) {
        f32x4* ac = acc[rb - 1];
#pragma unroll
        for (int cb = 0; cb < kF8CB; ++cb) asm volatile("" : "+v"(ac[cb]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    fm(NRB - 1);
  };
  Item it = decode_item_tiled(g, kF8Rows, kF8Groups, prefix, item);
  // A run: consecutive items of this workgroup with the same count of 16-row blocks
  // NRB (8, 7, 6, 5, 4 or 2; f8_item_blocks), computed by one body specialised on NRB,
  // so a partly filled tile does no matrix-core or rescale work for its padding.  Inside
  // a run the items are chained (CHAIN): the last chunk of an item loads, in place of
  // the clamped loads past its end, the next item's first chunk (written to LDS at that
  // chunk's end, so the next item starts on it), its second chunk (into the staging
  // registers) and its first two weight blocks (into the ring); the next item's
  // sorted_pair lookups are issued when an item starts and used at the end of its first
  // chunk.  The chained state never crosses the dispatch on NRB: a run's last item
  // loads its own data again in those places (dead loads, issued unconditionally), and
  // the next run starts by loading its first item's.  Without CHAIN a run is one item.
  auto run = [&](auto nrb) __attribute__((always_inline)) {
    constexpr int NRB = decltype(nrb)::value;
    int lk[kF8Loads + 1];
    F8Src ss;  // what the staging loads read: this item's, from its chunk NC - 2's end the next item's
    F8Src rs;  // what the weight ring loads: this item's, from its chunk NC - 1 the next item's
    F8Src nx;  // the next item's (the item's own again when the run ends with it)
    int par = 0;  // LDS buffer of the item's first chunk
    // the run's first item: its first chunk to LDS buffer 0, its second to the staging
    // registers, its first two weight blocks to the ring.  The first chunk's loads go out
    // before the ring's, so that the wait for them before their LDS write does not
    // include the ring's loads.
    f8_lookup(g, it, w, lane, lk);
    f8_source<SWIGLU>(g, it, w, lane, lk, ss);
    rs = ss;
    load_stage(ss, 0);
#pragma unroll
    for (int u = 0; u < kF8BAhead; ++u) load_ring(u, rs, u);
    write_stage(0);
    load_stage(ss, 1);
    __syncthreads();
    for (;;) {
      const int nitem = item + slots;
      const bool has_next = nitem < end;  // workgroup-uniform
      const Item nd = has_next ? decode_item_tiled(g, kF8Rows, kF8Groups, prefix, nitem) : it;
      const bool chain = CHAIN && has_next && f8_item_blocks(nd.nrows) == NRB;  // workgroup-uniform
      // field by field: a whole-struct copy moves its padding through scratch memory
      Item nit;
      nit.seg = chain ? nd.seg : it.seg;
      nit.shared = chain ? nd.shared : it.shared;
      nit.group = chain ? nd.group : it.group;
      nit.row0 = chain ? nd.row0 : it.row0;
      nit.nrows = chain ? nd.nrows : it.nrows;
      if (CHAIN) f8_lookup(g, nit, w, lane, lk);
      const int KB = (it.shared ? g.K_shared : g.K_routed) / 128;
      const int NC = (KB + 1) / 2;  // 256-deep chunks; an odd KB leaves the last chunk half live
      f32x4 acc[NRB][kF8CB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < kF8CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Chunk c computes from LDS buffer (c + par) % 2; at its end chunk c + 1 leaves the
      // staging registers for the other buffer, and they start loading chunk c + 2.
      // Chunk 0 runs outside the loop, so that the wait for the next item's lookups, at
      // its end, is on every path (else the compiler drains all loads where it reuses
      // their registers).
      auto chunk = [&](const int c) __attribute__((always_inline)) {
        const int buf = ((c + par) & 1) * kF8Buf;
        const bool ring_next = CHAIN && c == NC - 1;  // this chunk refills the ring with the next item's blocks
        if (ring_next) rs = nx;
        const int rbase = ring_next ? 2 * NC : 0;
        block(nrb, acc, 0, 0, buf);
        load_ring(0, rs, 2 * c + 2 - rbase);
        // issue the refill here, not after the next block's LDS traffic
        __builtin_amdgcn_sched_barrier(0);
        block(nrb, acc, 1, 1, buf);
        load_ring(1, rs, 2 * c + 3 - rbase);
        __builtin_amdgcn_sched_barrier(0);
        write_stage(kF8Buf - buf);
        __syncthreads();
        if (CHAIN && c == 0) f8_source<SWIGLU>(g, nit, w, lane, lk, nx);
        if (CHAIN && c == NC - 2) ss = nx;
        load_stage(ss, CHAIN && c >= NC - 2 ? c + 2 - NC : c + 2);
      };
      chunk(0);
      for (int c = 1; c < NC; ++c) chunk(c);
      f8_epilogue<SWIGLU, NRB>(g, it, w, lane, acc, qamax);
      par = (par + NC) & 1;
      it.seg = nd.seg;
      it.shared = nd.shared;
      it.group = nd.group;
      it.row0 = nd.row0;
      it.nrows = nd.nrows;
      item = nitem;
      if (!chain) break;
    }
  };
  // Each case of the dispatch ends in a distinct empty asm statement: the compiler would
  // otherwise merge the cases' common tails.
  while (item < end) {  // workgroup-uniform
    switch (f8_item_blocks(it.nrows)) {
      case 8: run(F8Blocks<8>{}); asm volatile("; 8 blocks"); break;
      case 7: run(F8Blocks<7>{}); asm volatile("; 7 blocks"); break;
      case 6: run(F8Blocks<6>{}); asm volatile("; 6 blocks"); break;
      case 5: run(F8Blocks<5>{}); asm volatile("; 5 blocks"); break;
      case 4: run(F8Blocks<4>{}); asm volatile("; 4 blocks"); break;
      default: run(F8Blocks<2>{}); asm volatile("; 2 blocks"); break;
    }
  }
}

template <bool SWIGLU, bool CHAIN>
static hipError_t launch_fp8_tiled(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = 2 * kF8Buf;  // above the default limit: see configure_gemm_fp8_tiled
  // max_blocks counts compute units; the kernel is built for kF8MinBlocks workgroups
  // on each
  const long long resident = (long long)max_blocks * kF8MinBlocks;
  long long blocks = max_items < resident ? max_items : resident;
  blocks = blocks < kF8Xcds ? kF8Xcds : blocks / kF8Xcds * kF8Xcds;
  gemm_fp8_tiled_kernel<SWIGLU, CHAIN><<<(unsigned)blocks, kF8Threads, smem, st>>>(g);
  return hipGetLastError();
}

// Reduction lengths are multiples of 128 and group counts multiples of 4 (the layer's
// dimensions are multiples of 128); output rows are 16-byte aligned (ldo % 4 == 0).
// Raise the kernels' dynamic LDS limit on the current device (handle creation).
hipError_t configure_gemm_fp8_tiled() {
  const int smem = 2 * kF8Buf;
  const void* fns[3] = {reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<true, false>),
                        reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<false, true>),
                        reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<false, false>)};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_fp8_tiled(const GroupedGemm& g, bool swiglu, long long a_rows, long long max_items,
                                 int max_blocks, hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  // item costs (at most 8 + kF8ItemFixedCost each) are summed in 32-bit ints
  if (max_items > 0x7fffffff / (kF8RowBlocks + kF8ItemFixedCost)) return hipErrorInvalidValue;
  if (g.K_routed % 128 || g.groups_routed % 4 || g.ldo_routed % 4 ||
      (g.shared_rows > 0 && (g.K_shared % 128 || g.groups_shared % 4 || g.ldo_shared % 4)))
    return hipErrorInvalidValue;
  // the quantising epilogue needs whole column tiles (every wave active)
  if (swiglu && g.outs_routed &&
      (g.groups_routed % kF8Groups || (g.shared_rows > 0 && g.groups_shared % kF8Groups)))
    return hipErrorInvalidValue;
  // activation rows are addressed by 32-bit byte offsets from the matrix's base
  if (a_rows < 0 || a_rows * g.lda_routed >= (1ll << 32) || (long long)g.shared_rows * g.lda_shared >= (1ll << 32))
    return hipErrorInvalidValue;
  if (swiglu) return launch_fp8_tiled<true, false>(g, max_items, max_blocks, st);
  // chained items need two chunks (K > 256) in every item
  const bool chain = g.K_routed > 256 && (g.shared_rows == 0 || g.K_shared > 256);
  return chain ? launch_fp8_tiled<false, true>(g, max_items, max_blocks, st)
               : launch_fp8_tiled<false, false>(g, max_items, max_blocks, st);
}

int fp8_tiled_rows() { return kF8Rows; }
int fp8_tiled_groups() { return kF8Groups; }

}  // namespace afd
