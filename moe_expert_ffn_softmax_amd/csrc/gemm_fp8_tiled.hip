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
// wave's MFMAs, and within a wave the instruction order interleaves them.  Each step rb of a block reads token block
// rb + 1's operand from LDS, then alternates block rb's MFMAs with the rescaling of
// block rb - 1's products (kept in a second register set).  The compiler would
// otherwise gather the pure arithmetic of the whole unrolled block in one place, so
// empty asm statements that consume a step's products and accumulators keep each step
// between scheduling barriers.
//
// For the gate/up projection the epilogue can write h already quantised (e4m3 codes
// and per-token per-128 scales; see below) instead of fp32 h.
//
// Items as in the bf16 tiled kernel; the XCD ranges carry equal costs (f8_xcd_range).
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
constexpr int kF8BAhead = 2;                    // scale blocks of weights in flight per wave
constexpr int kF8StageSets = 1;                 // chunks of activations loading ahead
constexpr int kF8LdsAhead = 1;                  // token blocks of operands read from LDS ahead
// The chunk loop is unrolled by two when a ring slot (block % kF8BAhead) or a staging
// set (chunk % kF8StageSets) would otherwise depend on the chunk's parity.
constexpr int kF8Unroll = (kF8BAhead == 4 || kF8StageSets == 2) ? 2 : 1;
constexpr int kF8Xcds = 8;

__device__ __forceinline__ f32x4 f8_mfma(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // scale operands 0: the compiler emits the unscaled v_mfma_f32_16x16x128_f8f6f4
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// A lane's 32 weight bytes of a packed fragment: 16 at p, 16 at p + 1 KiB.
__device__ __forceinline__ i32x8 f8_load32(const uint8_t* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  const i32x4 lo = q[0], hi = q[64];
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

constexpr int kF8MinBlocks = 1;  // workgroups per CU the registers must allow

// SiLU with the hardware reciprocal (one rounding more than z / (1 + e^-z)); h is
// quantised to e4m3 right after, whose step is 2^-3 of the value.
__device__ __forceinline__ float silu_rcp(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// One item: a tile of it.nrows <= 16 * NRB rows (NRB 16-row blocks hold all of them)
// times the workgroup's 8 column groups.  Blocks past NRB are not computed.
template <bool SWIGLU, int NRB>
__device__ __forceinline__ void fp8_tile(const GroupedGemm& g, const Item& it, const int w, unsigned char* lds,
                                         float (*qamax)[kF8Rows]) {
  // lane-derived indices are recomputed per item (hoisted out of the item loop they
  // do not fit the register budget)
  int lane = lane_id();
  asm volatile("" : "+v"(lane));
  const int K = it.shared ? g.K_shared : g.K_routed;
  const int KB = K / 128;
  const int NC = (KB + 1) / 2;  // 256-deep chunks; an odd KB leaves the last chunk half live
  const int groups = it.shared ? g.groups_shared : g.groups_routed;
  const int N = groups * 32;
  const int NB = N / 128;
  // A wave past the last group of a partial column tile recomputes the tile's last
  // two groups and stores nothing (group counts are multiples of 4).
  const bool active = it.group + w * kF8GroupsPerWave < groups;  // wave-uniform
  const int group0 = active ? it.group + w * kF8GroupsPerWave : groups - kF8GroupsPerWave;

  // staged rows: w*kF8StageRows + i*4 + lane/16 (i < kF8Loads); the lane loads piece
  // lane % 16 of each row's chunk
  const int lda = it.shared ? g.lda_shared : g.lda_routed;
  const uint8_t* abase = static_cast<const uint8_t*>(it.shared ? g.a_shared : g.a_routed);
  const int piece = lane & 15;
  // Source rows of the staged rows and of this thread's token-scale row (t % 128).
  // The sorted_pair lookups are
  // all issued before the first is used: in a branch per row, each would wait for
  // its load before the next one issues.
  int ar[kF8Loads + 1];
#pragma unroll
  for (int i = 0; i < kF8Loads; ++i) {
    const int r = w * kF8StageRows + i * 4 + (lane >> 4);
    ar[i] = it.row0 + (r < it.nrows ? r : 0);
  }
  {
    const int t = w * kF8StageRows + (lane & (kF8StageRows - 1));
    ar[kF8Loads] = it.row0 + (t < it.nrows ? t : 0);
  }
  if (!it.shared && g.gather_routed) {
#pragma unroll
    for (int i = 0; i <= kF8Loads; ++i) ar[i] = g.sorted_pair[ar[i]];
#pragma unroll
    for (int i = 0; i <= kF8Loads; ++i) ar[i] /= g.k;
  }
  const uint8_t* arow[kF8Loads];
#pragma unroll
  for (int i = 0; i < kF8Loads; ++i) arow[i] = abase + (size_t)ar[i] * lda;
  const float* asbase = it.shared ? g.as_shared : g.as_routed;
  const float* srow = asbase + (size_t)ar[kF8Loads] * KB;
  // byte offset in the row of chunk c's piece for this lane (clamped past the end of
  // K: that scale block is multiplied with weight scale 0)
  auto a_off = [&](int c) {
    const int o = c * 256 + piece * 16;
    return o < K ? o : o - 128;
  };
  // LDS: write slot of load i (token block (w*kF8StageRows + i*4 + lane/16) / 16 =
  // w*kF8StageRows/16 + i/4, slot = piece, row in block (i % 4) * 4 + lane / 16)
  const int wr_off = ((w * (kF8StageRows / 16)) * 16 + piece) * kF8Slot + (lane >> 4) * 16;
  // read: slot (lane / 16) * 2 (+1 for the upper 16 bytes) of the scale block's 8
  const int rd_off = ((lane >> 4) * 2) * kF8Slot + (lane & 15) * 16;

  const uint8_t* wbase = it.shared ? static_cast<const uint8_t*>(g.w_shared)
                                   : static_cast<const uint8_t*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
  const size_t group_stride = (size_t)KB * 4096;  // bytes per 32-column group
  // 16-column block cb = (group group0 + cb / 2, half cb % 2): 2 KiB per scale block
  const uint8_t* B = wbase + (size_t)group0 * group_stride + lane * 16;
  const float* ws = it.shared ? g.s_shared : g.s_routed + (size_t)it.seg * g.s_expert_elems;
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
  int wnb;
  {
    const int t = lane % (kF8WScales / 2);  // used by lanes >= 32
    const int w2 = t / kF8CB, cb = t % kF8CB;
    const int g0 = it.group + w2 * kF8GroupsPerWave < groups ? it.group + w2 * kF8GroupsPerWave
                                                             : groups - kF8GroupsPerWave;
    const int j = g0 + (cb >> 1), half = cb & 1;
    wnb = (SWIGLU ? half * (N / 2) + j * 16 : j * 32 + half * 16) / 128;
  }

  f32x4 acc[NRB][kF8CB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kF8CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging register sets: set (c % kF8StageSets) holds chunk c between its loads and
  // its LDS write.  Chunk 0 -> LDS buffer 0; chunks 1 .. kF8StageSets (clamped to the
  // last chunk) -> the sets.  Rows of token blocks past NRB are loaded (their rows
  // read the item's row 0) and written like the others, and never read.
  bf16x8 stage[kF8StageSets][kF8Loads];
  // sstage holds the lane's loaded scale and slive whether its block is inside K (a
  // block past the end of K, odd K / 128, gets weight scale 0): the zeroing is applied
  // when the value is written to LDS, so that no instruction needs the loaded value
  // before the write.
  float sstage[kF8StageSets];
  bool slive[kF8StageSets];
  auto load_stage = [&](const int set, int c) {
    c = c < NC ? c : NC - 1;
#pragma unroll
    for (int i = 0; i < kF8Loads; ++i) stage[set][i] = *reinterpret_cast<const bf16x8*>(arow[i] + a_off(c));
    const int kb = 2 * c + sc_blk;
    const int kbc = kb < KB ? kb : KB - 1;
    sstage[set] = *(sc_tok ? srow + kbc : ws + (size_t)kbc * NB + wnb);
    slive[set] = sc_tok || kb < KB;
  };
  auto write_stage = [&](const int set, int buf) {
#pragma unroll
    for (int i = 0; i < kF8Loads; ++i)
      *reinterpret_cast<bf16x8*>(lds + buf + wr_off + (i >> 2) * 16 * kF8Slot + (i & 3) * 64) = stage[set][i];
    *reinterpret_cast<float*>(lds + buf + sc_off) = slive[set] ? sstage[set] : 0.f;
  };
  // chunk 0's activations are loaded before the weight ring, so that the wait for
  // them before their LDS write does not include the ring's loads
  load_stage(0, 0);
  i32x8 bring[kF8BAhead][kF8CB];
#pragma unroll
  for (int u = 0; u < kF8BAhead; ++u) {
    const int s = u < KB ? u : KB - 1;
#pragma unroll
    for (int cb = 0; cb < kF8CB; ++cb) bring[u][cb] = f8_load32(B + (cb >> 1) * group_stride + (s * 2 + (cb & 1)) * 2048);
  }

  write_stage(0, 0);
#pragma unroll
  for (int u = 1; u <= kF8StageSets; ++u) load_stage(u % kF8StageSets, u);
  __syncthreads();

  // One 128-deep scale block: h is the block within the chunk, r its weight-ring slot
  // (block % kF8BAhead).
  auto block = [&](const int c, const int h, const int r, const int buf) {
    const int kb = 2 * c + h;
    const float* swl = reinterpret_cast<const float*>(lds + buf + kF8A) + 2 * kF8Rows +
                       h * (kF8WScales / 2) + w * kF8CB;
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
    auto rd = [&](const int rb) {
      const unsigned char* ap = lds + buf + (rb * 16 + h * 8) * kF8Slot + rd_off;
      const i32x4 l4 = *reinterpret_cast<const i32x4*>(ap);
      const i32x4 h4 = *reinterpret_cast<const i32x4*>(ap + kF8Slot);
      av[rb % (D + 1)] = i32x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
      sa[rb % (D + 2)] = sbuf[rb * 16];
    };
    auto fm = [&](const int rb) {
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
      if (rb + D < NRB) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int cb = 0; cb < kF8CB; ++cb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (rb > 0) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
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
    // refill this ring slot with the block kF8BAhead ahead (clamped to the last)
    int sn = kb + kF8BAhead;
    sn = sn < KB ? sn : KB - 1;
#pragma unroll
    for (int cb = 0; cb < kF8CB; ++cb)
      bring[r][cb] = f8_load32(B + (cb >> 1) * group_stride + (sn * 2 + (cb & 1)) * 2048);
    // issue the refill here, not after the chunk's staging writes (which wait for the
    // staging loads)
    __builtin_amdgcn_sched_barrier(0);
  };

  // Chunk c (parity u = c % 2 when unrolled) computes from LDS buffer c % 2; at its
  // end chunk c + 1 leaves its staging set for the other buffer, and that set starts
  // loading chunk c + 1 + kF8StageSets (clamped past the end; never consumed there).
  auto chunk = [&](const int c, const int u) {
    const int buf = u * kF8Buf;
    block(c, 0, (2 * u) % kF8BAhead, buf);
    block(c, 1, (2 * u + 1) % kF8BAhead, buf);
    const int set = (u + 1) % kF8StageSets;
    write_stage(set, kF8Buf - buf);
    __syncthreads();
    load_stage(set, c + 1 + kF8StageSets);
  };
  for (int c = 0; c < NC; c += kF8Unroll) {
    if (kF8Unroll == 1) {
      chunk(c, c & 1);
    } else {
      chunk(c, 0);
      if (c + 1 < NC) chunk(c + 1, 1);
    }
  }

  float* qscale = it.shared ? g.outs_shared : g.outs_routed;
  if (SWIGLU && qscale) {
    // h quantised in place of the separate pass: the tile's 8 groups are exactly one
    // 128-channel quantisation group of each of its tokens (gate/up column tiles are
    // whole, as 2M/32 is a multiple of 8).  Per token: amax over the 4 lanes of
    // each wave holding it, then over the 4 waves through LDS; scale = amax / 448
    // (1 for an all-zero group); codes = e4m3(v * (1 / scale)) with the reciprocal
    // rounded once per token group, one rounding more than the quantisation kernel's
    // e4m3(v / scale), and SiLU through the hardware reciprocal: h is internal to
    // the layer, and its codes may differ from the streaming path's by one step.
    const int tok = lane & 15;
    const int n0 = (lane >> 4) * 4;
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
  } else if (active) {
    const int tok = lane & 15;
    const int n0 = (lane >> 4) * 4;
    float* out = static_cast<float*>(it.shared ? g.out_shared : g.out_routed);
    const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int t = rb * 16 + tok;
      if (t >= it.nrows) continue;
      float* o = out + (size_t)(it.row0 + t) * ldo;
#pragma unroll
      for (int j = 0; j < kF8GroupsPerWave; ++j) {
        if (SWIGLU) {
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

template <bool SWIGLU>
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

  for (int item = begin + slot; item < end; item += slots) {
    const Item it = decode_item_tiled(g, kF8Rows, kF8Groups, prefix, item);
    // the item's computation is specialised on its count of 16-row blocks, so the
    // padding of a partly filled tile costs neither matrix-core nor rescaling work
    const int nb = f8_item_blocks(it.nrows);  // wave-uniform
    if (nb == 8)
      fp8_tile<SWIGLU, 8>(g, it, w, lds, qamax);
    else if (nb == 7)
      fp8_tile<SWIGLU, 7>(g, it, w, lds, qamax);
    else if (nb == 6)
      fp8_tile<SWIGLU, 6>(g, it, w, lds, qamax);
    else if (nb == 5)
      fp8_tile<SWIGLU, 5>(g, it, w, lds, qamax);
    else if (nb == 4)
      fp8_tile<SWIGLU, 4>(g, it, w, lds, qamax);
    else
      fp8_tile<SWIGLU, 2>(g, it, w, lds, qamax);
    // every LDS read of this item happened before its last chunk's barrier
  }
}

template <bool SWIGLU>
static hipError_t launch_fp8_tiled(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = 2 * kF8Buf;  // above the default limit: see configure_gemm_fp8_tiled
  // max_blocks counts compute units; the kernel is built for kF8MinBlocks workgroups
  // on each
  const long long resident = (long long)max_blocks * kF8MinBlocks;
  long long blocks = max_items < resident ? max_items : resident;
  blocks = blocks < kF8Xcds ? kF8Xcds : blocks / kF8Xcds * kF8Xcds;
  gemm_fp8_tiled_kernel<SWIGLU><<<(unsigned)blocks, kF8Threads, smem, st>>>(g);
  return hipGetLastError();
}

// Reduction lengths are multiples of 128 and group counts multiples of 4 (the layer's
// dimensions are multiples of 128); output rows are 16-byte aligned (ldo % 4 == 0).
// Raise the kernels' dynamic LDS limit on the current device (handle creation).
hipError_t configure_gemm_fp8_tiled() {
  const int smem = 2 * kF8Buf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_fp8_tiled_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  return e;
}

hipError_t launch_gemm_fp8_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                 hipStream_t st) {
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
  return swiglu ? launch_fp8_tiled<true>(g, max_items, max_blocks, st) : launch_fp8_tiled<false>(g, max_items, max_blocks, st);
}

int fp8_tiled_rows() { return kF8Rows; }
int fp8_tiled_groups() { return kF8Groups; }

}  // namespace afd
