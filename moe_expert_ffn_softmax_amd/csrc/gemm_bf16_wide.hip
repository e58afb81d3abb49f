// Grouped expert GEMMs in bf16, 256x256 tiles, for batches whose experts receive
// hundreds of rows (the aggregated FFN-instance batches of "大模型推理的内存与计算解耦：
// AFD 架构解析与性能验证", §2, and MegaScale-Infer in "AF分离论文串讲"; there the
// expert GEMMs are compute-bound: the omica.com.cn AFD article, §2.1).
//
// Why a second large-tile kernel.  Past ~300 rows per expert the layer is bound by
// the matrix cores, and what feeds them is the path L2 -> L1 -> registers.  A 128 x
// 256 tile moves 384 bytes through it per unit of reduction depth for 32768 FLOP; a
// 256 x 256 tile moves 512 bytes for 65536, a third less per FLOP, and each weight
// fragment is then used for 256 rows inside the workgroup instead of relying on the
// L2 to serve the next row tile (measured: the 128-row kernel missed L2 on ~40% of
// its requests at 1024 rows per expert, this one on ~25%).  The price is LDS traffic:
// both operands are written to and read from LDS, 768 bytes per MFMA against 640 for
// the 128-row kernel, and on MI355X the LDS writes cost the MFMA loop about a quarter
// of its rate.  Measured end to end it is no faster than the 128-row kernel, so it is
// selected only on request (a tuning and testing option).
//
// Workgroup: 4 waves in a 2 x 2 arrangement; wave (wm, wn) owns rows wm*128 .. +127
// and the item's 32-column groups wn*4 .. +3, i.e. 4 x 4 blocks of 32 x 32, one
// v_mfma_f32_32x32x16_bf16 accumulator each (256 accumulator registers).  Both
// operands go through LDS, 64 reduction rows (one chunk) at a time, double-buffered:
// the next chunk is loaded into registers while the current one is multiplied, then
// written to the other buffer before the chunk's last barrier.  Inside a chunk the
// operands of the next 16-deep half-step are read while the current half-step's 16
// MFMAs run.
//
// LDS layout of one buffer:
//  * A: 8 row blocks x 4 fragments (16-deep halves of the chunk's two 32-deep steps);
//    a fragment holds lane l' (row l' % 32, reduction half l' / 32) at byte
//    (l' % 32) * 16 + (l' / 32) * 528 of a 1056-byte slot.  A row arrives as 8
//    16-byte pieces (4 fragments x 2 halves) from 8 lanes: with this padding they
//    fall on 8 different 16-byte bank groups, and the two rows of one 16-lane
//    quarter are 8 rows apart, so they use the other 8 groups.  Fragment reads stay
//    contiguous per 8- and 16-lane part.  Rows are loaded 8 per instruction, 128
//    contiguous bytes each.
//  * B: the packed weight fragments of the 8 groups x 2 steps, copied verbatim (the
//    packed order is already the operand order); 2 KiB per (group, step).
//
// Operand and SwiGLU conventions are those of the 128-row kernel: lane l supplies row
// (l % 32) of A and column (l % 32) of B at reduction offsets (l / 32) * 8 .. + 7 and
// receives rows (i / 4) * 8 + (l / 32) * 4 + i % 4 of column (l % 32); for the
// gate/up projection block 2p holds the gate and block 2p + 1 the up columns of the
// same 32 intermediate channels.  Items are (segment, column tile, row tile), row
// tile fastest, cut into 8 contiguous ranges, one per XCD.
#include "grouped.h"

namespace afd {

typedef float f32x16w __attribute__((ext_vector_type(16)));

constexpr int kWideWaves = 4;
constexpr int kWideThreads = kWideWaves * kWave;
constexpr int kWideRows = 256;
constexpr int kWideGroups = 8;                          // 32-column groups per item
constexpr int kWideRB = 4;                              // 32-row blocks per wave
constexpr int kWideCB = 4;                              // 32-column blocks per wave
constexpr int kWideFrags = 4;                           // 16-deep fragments per chunk (64 deep)
constexpr int kWideSlot = 1056;                         // A fragment slot bytes (1 KiB + padding)
constexpr int kWideHalf = 528;                          // byte offset of reduction half 1 in a slot
constexpr int kWideA = 8 * kWideFrags * kWideSlot;      // A bytes per buffer (8 row blocks)
constexpr int kWideB = kWideGroups * 2 * 2048;          // B bytes per buffer (8 groups x 2 steps)
constexpr int kWideBuf = kWideA + kWideB;
constexpr int kWideLoads = 8;                           // A and B staging loads per thread per chunk
constexpr int kWideXcds = 8;

#ifndef AFD_WIDE_SCHED
#define AFD_WIDE_SCHED 1
#endif

template <bool SWIGLU>
__global__ void __launch_bounds__(kWideThreads, 1) gemm_bf16_wide_kernel(GroupedGemm g) {
  __shared__ int prefix[kMaxSegments + 1];
  __shared__ int scan_tmp[kWideWaves + 1];
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int total = build_item_prefix(g, kWideRows, kWideGroups, prefix, scan_tmp);
  const int w = threadIdx.x / kWave;
  const int wm = w >> 1, wn = w & 1;

  const int xcd = blockIdx.x % kWideXcds;
  const int slot = blockIdx.x / kWideXcds;
  const int slots = gridDim.x / kWideXcds;
  const int begin = (int)((long long)total * xcd / kWideXcds);
  const int end = (int)((long long)total * (xcd + 1) / kWideXcds);

  for (int item = begin + slot; item < end; item += slots) {
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const Item it = decode_item_tiled(g, kWideRows, kWideGroups, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 32;
    const int NC = K / 64;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    // Group counts are multiples of 4, so a wave's 4 groups are all valid or all past
    // the end of a partial column tile; such a wave (and the staging of its groups)
    // repeats the tile's previous 4 groups and stores nothing.
    const bool active = it.group + wn * 4 < groups;  // wave-uniform

    // A staging: instruction i = 2a + b carries rows w*64 + a*16 + b*4 + ro(lane/8)
    // with ro(q) = q/2 + (q%2)*8 (two rows 8 apart per 16-lane quarter), 16-byte piece
    // lane%8 of the row's 128-byte chunk slice
    const int lda = it.shared ? g.lda_shared : g.lda_routed;
    const __bf16* abase = static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed);
    const int piece = lane & 7;
    const bf16x8* arow[kWideLoads];
#pragma unroll
    for (int i = 0; i < kWideLoads; ++i) {
      const int q = lane >> 3;
      int r = w * 64 + (i >> 1) * 16 + (i & 1) * 4 + (q >> 1) + (q & 1) * 8;
      r = r < it.nrows ? r : 0;
      int ar;
      if (it.shared)
        ar = it.row0 + r;
      else
        ar = g.gather_routed ? g.sorted_pair[it.row0 + r] / g.k : it.row0 + r;
      arow[i] = reinterpret_cast<const bf16x8*>(abase + (size_t)ar * lda) + piece;
    }
    // B staging: load j copies unit threadIdx.x of group j's 2 steps of the chunk (the
    // group bases are workgroup-uniform; only the unit offset is per lane)
    const bf16x8* wbase = reinterpret_cast<const bf16x8*>(
        it.shared ? static_cast<const __bf16*>(g.w_shared)
                  : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems);
    const int glast = groups - it.group;  // groups of this column tile (4 or >= 8)
    auto bsrc = [&](int j, int cn) {
      const int gi = it.group + (j < glast ? j : j - 4);
      return wbase + ((size_t)gi * KB * 128 + cn * 256) + threadIdx.x;
    };

    // LDS offsets (bytes)
    const int a_ro = ((lane >> 3) >> 1) + ((lane >> 3) & 1) * 8;
    const int a_wr = ((w * 2) * kWideFrags + (piece >> 1)) * kWideSlot + a_ro * 16 + (piece & 1) * kWideHalf;
    const int a_rd = (wm * kWideRB * kWideFrags) * kWideSlot + (lane & 31) * 16 + (lane >> 5) * kWideHalf;
    int b_rd[kWideCB];
#pragma unroll
    for (int cb = 0; cb < kWideCB; ++cb) {
      const int grp = SWIGLU ? wn * 4 + (cb >> 1) * 2 + ((lane & 31) >> 4) : wn * 4 + cb;
      const int half = SWIGLU ? (cb & 1) : ((lane & 31) >> 4);
      b_rd[cb] = kWideA + ((grp * 2) * 128 + half * 64 + (lane >> 5) * 16 + (lane & 15)) * 16;
    }

    f32x16w acc[kWideRB][kWideCB];
#pragma unroll
    for (int rb = 0; rb < kWideRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kWideCB; ++cb) acc[rb][cb] = f32x16w{};

    // chunk 0 -> LDS buffer 0; chunk 1 (or 0 again) -> staging registers
    bf16x8 sa[kWideLoads], sb[kWideLoads];
#pragma unroll
    for (int i = 0; i < kWideLoads; ++i) {
      sa[i] = arow[i][0];
      sb[i] = *bsrc(i, 0);
    }
#pragma unroll
    for (int i = 0; i < kWideLoads; ++i) {
      *reinterpret_cast<bf16x8*>(lds + a_wr + ((i >> 1) >> 1) * kWideFrags * kWideSlot + (((i >> 1) & 1) * 16 + (i & 1) * 4) * 16) = sa[i];
      *reinterpret_cast<bf16x8*>(lds + kWideA + (i * kWideThreads + threadIdx.x) * 16) = sb[i];
    }
    {
      const int cn = NC > 1 ? 1 : 0;
#pragma unroll
      for (int i = 0; i < kWideLoads; ++i) {
        sa[i] = arow[i][cn * 8];
        sb[i] = *bsrc(i, cn);
      }
    }
    __syncthreads();

    bf16x8 a[2][kWideRB], b[2][kWideCB];
#pragma unroll
    for (int rb = 0; rb < kWideRB; ++rb)
      a[0][rb] = *reinterpret_cast<const bf16x8*>(lds + a_rd + rb * kWideFrags * kWideSlot);
#pragma unroll
    for (int cb = 0; cb < kWideCB; ++cb) b[0][cb] = *reinterpret_cast<const bf16x8*>(lds + b_rd[cb]);

    for (int c = 0; c < NC; ++c) {
      const int buf = (c & 1) * kWideBuf;
      const int nbuf = kWideBuf - buf;
#pragma unroll
      for (int hs = 0; hs < kWideFrags; ++hs) {
        const int cur = hs & 1, nxt = cur ^ 1;
        if (hs + 1 < kWideFrags) {
          // fragment hs+1 = (step (hs+1)/2, half (hs+1)%2)
          const int f = hs + 1;
#pragma unroll
          for (int rb = 0; rb < kWideRB; ++rb)
            a[nxt][rb] = *reinterpret_cast<const bf16x8*>(lds + buf + a_rd + (rb * kWideFrags + f) * kWideSlot);
#pragma unroll
          for (int cb = 0; cb < kWideCB; ++cb)
            b[nxt][cb] = *reinterpret_cast<const bf16x8*>(lds + buf + b_rd[cb] + ((f >> 1) * 128 + (f & 1) * 32) * 16);
        } else {
          // branch-free chunk boundary: past the last chunk these write, load and read
          // data nobody uses (the loads are clamped to the last chunk)
#pragma unroll
          for (int i = 0; i < kWideLoads; ++i) {
            *reinterpret_cast<bf16x8*>(lds + nbuf + a_wr + ((i >> 1) >> 1) * kWideFrags * kWideSlot + (((i >> 1) & 1) * 16 + (i & 1) * 4) * 16) = sa[i];
            *reinterpret_cast<bf16x8*>(lds + nbuf + kWideA + (i * kWideThreads + threadIdx.x) * 16) = sb[i];
          }
          __syncthreads();
          const int cn = c + 2 < NC ? c + 2 : NC - 1;
#pragma unroll
          for (int i = 0; i < kWideLoads; ++i) {
            sa[i] = arow[i][cn * 8];
            sb[i] = *bsrc(i, cn);
          }
#pragma unroll
          for (int rb = 0; rb < kWideRB; ++rb)
            a[nxt][rb] = *reinterpret_cast<const bf16x8*>(lds + nbuf + a_rd + rb * kWideFrags * kWideSlot);
#pragma unroll
          for (int cb = 0; cb < kWideCB; ++cb) b[nxt][cb] = *reinterpret_cast<const bf16x8*>(lds + nbuf + b_rd[cb]);
        }
#pragma unroll
        for (int rb = 0; rb < kWideRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < kWideCB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][rb], b[cur][cb], acc[rb][cb], 0, 0, 0);
#if AFD_WIDE_SCHED
        // spread the next half-step's 8 LDS reads between this half-step's 16 MFMAs
#pragma unroll
        for (int q = 0; q < kWideRB + kWideCB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
        }
#endif
      }
    }

    if (active) {
      const int col = lane & 31;
      const int rsub = wm * 128 + (lane >> 5) * 4;
      const int g0 = it.group + wn * 4;
      if (SWIGLU) {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kWideRB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rsub + rb * 32 + (i / 4) * 8 + (i % 4);
            if (row < it.nrows) {
              __bf16* o = out + (size_t)(it.row0 + row) * ldo + g0 * 16 + col;
              o[0] = f32_to_bf16(silu(acc[rb][0][i]) * acc[rb][1][i]);
              o[32] = f32_to_bf16(silu(acc[rb][2][i]) * acc[rb][3][i]);
            }
          }
      } else {
        __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
        const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
        for (int rb = 0; rb < kWideRB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = rsub + rb * 32 + (i / 4) * 8 + (i % 4);
            if (row < it.nrows) {
              __bf16* o = out + (size_t)(it.row0 + row) * ldo + g0 * 32 + col;
#pragma unroll
              for (int cb = 0; cb < kWideCB; ++cb) o[cb * 32] = f32_to_bf16(acc[rb][cb][i]);
            }
          }
      }
    }
    // every LDS read of this item was issued before the barrier of its last half-step
  }
}

template <bool SWIGLU>
static hipError_t launch_wide(const GroupedGemm& g, long long max_items, int max_blocks, hipStream_t st) {
  const size_t smem = 2 * kWideBuf;  // above the default limit: see configure_gemm_bf16_wide
  long long blocks = max_items < max_blocks ? max_items : max_blocks;
  blocks = blocks < kWideXcds ? kWideXcds : blocks / kWideXcds * kWideXcds;
  gemm_bf16_wide_kernel<SWIGLU><<<(unsigned)blocks, kWideThreads, smem, st>>>(g);
  return hipGetLastError();
}

// Reduction lengths are multiples of 128 and group counts multiples of 4 (the layer's
// dimensions are multiples of 128); `max_blocks` counts compute units.
// Raise the kernels' dynamic LDS limit on the current device (handle creation).
hipError_t configure_gemm_bf16_wide() {
  const int smem = 2 * kWideBuf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_wide_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_wide_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  return e;
}

hipError_t launch_gemm_bf16_wide(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                 hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  if (g.K_routed % 64 || g.groups_routed % 4 || (g.shared_rows > 0 && (g.K_shared % 64 || g.groups_shared % 4)))
    return hipErrorInvalidValue;
  return swiglu ? launch_wide<true>(g, max_items, max_blocks, st) : launch_wide<false>(g, max_items, max_blocks, st);
}

int wide_rows() { return kWideRows; }
int wide_groups() { return kWideGroups; }

}  // namespace afd
