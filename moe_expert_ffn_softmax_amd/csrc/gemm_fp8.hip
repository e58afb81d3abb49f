// Grouped expert GEMMs with fp8 (OCP e4m3) operands and fp32 block scales on the
// gfx950 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales).
//
// Weights carry one fp32 scale per 128x128 block and activations one per row per
// 128 channels, so every 128-deep reduction block of an output element has exactly
// one scale on each side: one MFMA instruction covers one such block, and its fp32
// partial product is added to the accumulator times s_act[row][kb] * s_w[kb][nb]
// (the FP8 DeepGEMM of "大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §1, is
// NVIDIA prior art with the same block structure; FP8/BF16 mixed precision is the
// omica.com.cn AFD article's §3.3).
//
// Operand order.  A fragment is 64 lanes x 32 bytes: lane l supplies row (l % 16) of
// A and column (l % 16) of B at reduction offsets (l / 16) * 32 .. + 31 of the
// 128-deep block.  The instruction pairs A and B bytes held in the same (lane group,
// register, byte) position, so any packing used identically on both sides gives the
// exact block dot product; this one keeps each lane's 32 bytes contiguous in a row of
// x (two 16-byte loads).  The result layout is that of the 16x16 fp32 MFMAs: lane l
// holds rows (l / 16) * 4 .. + 3 of column (l % 16).
//
// Work items, weight streaming and item striding are those of the bf16 streaming
// kernel: one wave per 16-row tile times one 32-column group, full reduction,
// weight fragments (and the blocks' scales) loaded nontemporally four blocks ahead.
#include "grouped.h"

namespace afd {

constexpr int kFp8Threads = 256;
constexpr int kFp8Waves = kFp8Threads / kWave;

__device__ __forceinline__ f32x4 mfma_fp8_block(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // format codes 0 (fp8 e4m3) for both operands, E8M0 scale 127 = 2^0 on both sides
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// A lane's 32 weight bytes of a packed fragment: 16 at p, 16 at p + 1 KiB (see the
// packing below).
__device__ __forceinline__ i32x8 load_frag_nt(const uint8_t* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  const i32x4 lo = __builtin_nontemporal_load(q), hi = __builtin_nontemporal_load(q + 64);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ i32x8 load32(const uint8_t* p) {
  const i32x4* q = reinterpret_cast<const i32x4*>(p);
  const i32x4 lo = q[0], hi = q[1];
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Column of the first element of packed 16-column block (group j, half) of a matrix
// with N output columns.
__device__ __forceinline__ int block_col(bool gate_up, int N, int j, int half) {
  return gate_up ? half * (N / 2) + j * 16 : j * 32 + half * 16;
}

// acc0/acc1 += the 128-deep blocks 0..KB-1 of one 16-row tile and two 16-column weight
// blocks, each block's fp32 product rescaled by s_act[row][kb] * s_w[kb][nb].  A ring of
// D blocks in flight holds the operands and the block's scales (two weight scales,
// the activation scales of the lane's four rows), so a block waits on no load issued
// in its own iteration; no branch inside (KB % D == 0, KB >= D), so the compiler
// waits only for the oldest loads.  The weight half of the first D blocks is loaded
// first (fp8_prime_weights), before the activation rows are known.
template <int D>
struct Fp8Ring {
  i32x8 a[D], b0[D], b1[D];
  float w0r[D], w1r[D], sar[D][4];
};

template <int D>
__device__ __forceinline__ void fp8_fetch_w(Fp8Ring<D>& r, const uint8_t* __restrict__ B,
                                            const float* __restrict__ ws, int NB, int nb0, int nb1, int u, int kb) {
  r.b0[u] = load_frag_nt(B + (kb * 2) * 2048);
  r.b1[u] = load_frag_nt(B + (kb * 2 + 1) * 2048);
  r.w0r[u] = ws[(size_t)kb * NB + nb0];
  r.w1r[u] = ws[(size_t)kb * NB + nb1];
}

template <int D>
__device__ __forceinline__ void fp8_fetch_a(Fp8Ring<D>& r, const uint8_t* __restrict__ A,
                                            const float* const (&as_row)[4], int u, int kb) {
  r.a[u] = load32(A + kb * 128);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.sar[u][i] = as_row[i][kb];
}

template <int D>
__device__ __forceinline__ void fp8_prime_weights(Fp8Ring<D>& r, const uint8_t* __restrict__ B,
                                                  const float* __restrict__ ws, int NB, int nb0, int nb1) {
#pragma unroll
  for (int u = 0; u < D; ++u) fp8_fetch_w(r, B, ws, NB, nb0, nb1, u, u);
}

template <int D>
__device__ __forceinline__ void stream_fp8_primed(Fp8Ring<D>& r, const uint8_t* __restrict__ A,
                                                  const uint8_t* __restrict__ B, const float* __restrict__ ws,
                                                  int NB, int nb0, int nb1, const float* const (&as_row)[4], int KB,
                                                  f32x4& acc0, f32x4& acc1) {
  auto compute = [&](const int u) {
    const f32x4 p0 = mfma_fp8_block(r.a[u], r.b0[u]);
    const f32x4 p1 = mfma_fp8_block(r.a[u], r.b1[u]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0[i] = fmaf(p0[i], r.sar[u][i] * r.w0r[u], acc0[i]);
      acc1[i] = fmaf(p1[i], r.sar[u][i] * r.w1r[u], acc1[i]);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) fp8_fetch_a(r, A, as_row, u, u);
  for (int kb0 = D; kb0 < KB; kb0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      compute(u);
      fp8_fetch_a(r, A, as_row, u, kb0 + u);
      fp8_fetch_w(r, B, ws, NB, nb0, nb1, u, kb0 + u);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) compute(u);
}

// One item's reduction: the weight half of the ring's first blocks, then the activation
// rows (rows[], or the rows behind pairs[] when the tile is gathered), then the stream.
template <int D>
__device__ __forceinline__ void fp8_stream_item(const GroupedGemm& g, const Item& it, int lane, int (&rows)[5],
                                                const int (&pairs)[5], const uint8_t* __restrict__ B,
                                                const float* __restrict__ ws, int NB, int nb0, int nb1, int KB,
                                                f32x4& acc0, f32x4& acc1) {
  Fp8Ring<D> ring;
  fp8_prime_weights<D>(ring, B, ws, NB, nb0, nb1);
  __builtin_amdgcn_sched_barrier(0);  // the weight loads issue before the entries are used
  if (!it.shared && g.gather_routed) {
#pragma unroll
    for (int i = 0; i < 5; ++i) rows[i] = pairs[i] / g.k;
  }
  const int lda = it.shared ? g.lda_shared : g.lda_routed;
  const uint8_t* A = static_cast<const uint8_t*>(it.shared ? g.a_shared : g.a_routed) + (size_t)rows[0] * lda +
                     (lane >> 4) * 32;
  const float* as_base = it.shared ? g.as_shared : g.as_routed;
  const float* as_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) as_row[i] = as_base + (size_t)rows[1 + i] * KB;
  stream_fp8_primed<D>(ring, A, B, ws, NB, nb0, nb1, as_row, KB, acc0, acc1);
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kFp8Threads) gemm_fp8_stream_kernel(GroupedGemm g) {
  __shared__ SegTable prefix;
  __shared__ int scan_tmp[kFp8Waves + 1];
  const int total = build_item_prefix(g, kTileRows, prefix, scan_tmp);
  const int lane = lane_id();
  const int waves_in_launch = gridDim.x * kFp8Waves;
  const int wave = blockIdx.x * kFp8Waves + threadIdx.x / kWave;

  for (int item = wave; item < total; item += waves_in_launch) {
    const Item it = decode_item(g, kTileRows, prefix, item);
    const int K = it.shared ? g.K_shared : g.K_routed;
    const int KB = K / 128;
    const int groups = it.shared ? g.groups_shared : g.groups_routed;
    const int N = groups * 32;
    const int NB = N / 128;  // weight scale blocks per reduction block
    // Rows of this lane: its A row (tile row lane % 16) and the 4 output rows whose
    // activation scales it applies (rows past the tile end repeat its first row).
    // Their sorted_pair entries are loaded first (in-bounds entries are read for every
    // tile, used only when the tile's rows are gathered), then the weight half of the
    // first ring blocks, so that the wait for the entries does not include the weights.
    const int r = lane & 15;
    int rows[5];
    rows[0] = it.row0 + (r < it.nrows ? r : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int orow = (lane >> 4) * 4 + i;
      rows[1 + i] = it.row0 + (orow < it.nrows ? orow : 0);
    }
    int pairs[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) pairs[i] = g.sorted_pair[rows[i]];
    const uint8_t* wbase = it.shared ? static_cast<const uint8_t*>(g.w_shared)
                                     : static_cast<const uint8_t*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
    const uint8_t* B = wbase + (size_t)it.group * KB * 4096 + lane * 16;  // [kb][half][2][lane][16 B]
    const float* ws = it.shared ? g.s_shared : g.s_routed + (size_t)it.seg * g.s_expert_elems;
    const int nb0 = block_col(SWIGLU, N, it.group, 0) / 128, nb1 = block_col(SWIGLU, N, it.group, 1) / 128;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (KB % 4 == 0)
      fp8_stream_item<4>(g, it, lane, rows, pairs, B, ws, NB, nb0, nb1, KB, acc0, acc1);
    else if (KB % 2 == 0)
      fp8_stream_item<2>(g, it, lane, rows, pairs, B, ws, NB, nb0, nb1, KB, acc0, acc1);
    else
      fp8_stream_item<1>(g, it, lane, rows, pairs, B, ws, NB, nb0, nb1, KB, acc0, acc1);

    const int col = lane & 15;
    const int rbase = (lane >> 4) * 4;
    const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rbase + i;
      if (row >= it.nrows) continue;
      if (SWIGLU) {
        // fp32 h, quantised by the next pass
        float* o = static_cast<float*>(it.shared ? g.out_shared : g.out_routed) + (size_t)(it.row0 + row) * ldo;
        o[it.group * 16 + col] = silu(acc0[i]) * acc1[i];
      } else {
        __bf16* o = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed) + (size_t)(it.row0 + row) * ldo;
        o[it.group * 32 + col] = f32_to_bf16(acc0[i]);
        o[it.group * 32 + 16 + col] = f32_to_bf16(acc1[i]);
      }
    }
  }
}

hipError_t launch_gemm_fp8(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  long long blocks = (max_items + kFp8Waves - 1) / kFp8Waves;
  if (blocks > max_blocks) blocks = max_blocks;
  if (swiglu)
    gemm_fp8_stream_kernel<true><<<(unsigned)blocks, kFp8Threads, 0, st>>>(g);
  else
    gemm_fp8_stream_kernel<false><<<(unsigned)blocks, kFp8Threads, 0, st>>>(g);
  return hipGetLastError();
}

hipError_t gemm_occupancy_fp8(int* gate_up, int* down) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(gate_up, gemm_fp8_stream_kernel<true>, kFp8Threads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(down, gemm_fp8_stream_kernel<false>, kFp8Threads, 0);
  return e;
}

// Repack fp8 weights [nmat][R][C] into 2 KiB fragments [group][kb][half], each
// holding lane l's 32 reduction bytes as two 16-byte halves at l * 16 and 1024 + l * 16,
// so that each of the two loads of a fragment reads 1 KiB contiguously (group/half
// pairing as for bf16).
__global__ void pack_fp8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int nmat, int R, int C,
                                int gate_up) {
  const size_t slots_per_mat = (size_t)R * C / 32;
  const size_t total = slots_per_mat * nmat;
  const int KB = R / 128;
  for (size_t s = blockIdx.x * (size_t)blockDim.x + threadIdx.x; s < total; s += (size_t)gridDim.x * blockDim.x) {
    const size_t mat = s / slots_per_mat;
    size_t rem = s % slots_per_mat;
    const int lane = (int)(rem % 64);
    rem /= 64;
    const int half = (int)(rem % 2);
    rem /= 2;
    const int kb = (int)(rem % KB);
    const int j = (int)(rem / KB);
    const int c = lane % 16;
    const int col = gate_up ? half * (C / 2) + j * 16 + c : j * 32 + half * 16 + c;
    const int row0 = kb * 128 + (lane / 16) * 32;
    const uint8_t* sp = src + mat * (size_t)R * C + (size_t)row0 * C + col;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (uint32_t)sp[(size_t)(4 * i) * C] | ((uint32_t)sp[(size_t)(4 * i + 1) * C] << 8) |
             ((uint32_t)sp[(size_t)(4 * i + 2) * C] << 16) | ((uint32_t)sp[(size_t)(4 * i + 3) * C] << 24);
    uint8_t* frag = dst + (s / 64) * 2048 + lane * 16;
    uint32_t* lo = reinterpret_cast<uint32_t*>(frag);
    uint32_t* hi = reinterpret_cast<uint32_t*>(frag + 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = w[i];
      hi[i] = w[4 + i];
    }
  }
}

hipError_t launch_pack_fp8(const uint8_t* src, uint8_t* dst, int nmat, int R, int C, int gate_up, hipStream_t st) {
  if (R % 128 || C % 32) return hipErrorInvalidValue;
  pack_fp8_kernel<<<4096, 256, 0, st>>>(src, dst, nmat, R, C, gate_up);
  return hipGetLastError();
}

}  // namespace afd
