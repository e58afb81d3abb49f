// Measurement probes of what MI355X (gfx950) attains on the two resources the layer's
// GEMMs are bound by, for reading the kernels' roofline fractions against something
// measured as well as the published peaks.  Not part of the layer: built into its own
// library (libafd_probe.so) and driven by bench.py --attainable.
//
//   afd_probe_stream: HBM reads in the weight-streaming GEMM's pattern: `runs` private
//     runs of `run_bytes` each, one wave per run, 16-byte nontemporal loads that cover
//     1 KiB per wave per step, `depth` steps in flight in a register ring.  Each lane
//     adds what it read (32-bit wrap-around) and stores the sum, so the result can be
//     checked against the buffer's sum.
//   afd_probe_mfma: back-to-back matrix-core instructions on operands drawn at random
//     (eight independent accumulators per wave, each with its own operands): kind 0 is
//     v_mfma_f32_32x32x16_bf16, kind 1 v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3).
//   afd_probe_lds: LDS reads in the tiled GEMMs' operand pattern (16-byte reads, each
//     16-lane quarter of a wave reading one contiguous 256-byte slot), 8 waves per
//     compute unit; reports each wave's cycle count.
//   afd_probe_fp8_block: the fp8 tiled GEMM's inner loop without global memory, on
//     random operands, 8 waves per workgroup (two per SIMD), each with 8 token blocks x
//     2 weight column blocks, two v_mfma_f32_16x16x128_f8f6f4 per token block.  mode 0:
//     the instructions accumulate directly; mode 1: their products are added to the
//     accumulators times a per-token, per-column-block scale (one multiply and four
//     FMAs per instruction, the previous token block's while the current one's
//     instructions run), token operands in registers; mode 2: as 1, token operands read
//     from LDS one token block ahead, in the GEMM's slot layout; mode 3: as 2, plus,
//     every two scale blocks, the staging writes of a chunk (four 16-byte and one
//     4-byte LDS write per thread) and a workgroup barrier.  Reports each wave's cycles.
//   afd_probe_bf16_block: the bf16 tiled GEMM's inner loop without global memory: 4
//     waves per workgroup (one per SIMD), each with 4 row blocks of 32 x 2 column blocks
//     of 32, v_mfma_f32_32x32x16_bf16 accumulating directly, 64 per wave per 128-deep
//     chunk.  mode 0: operands in registers; mode 1: the row blocks' operands read from
//     LDS in the GEMM's fragment layout; mode 2: as 1, plus a chunk's staging writes
//     (eight 16-byte LDS writes per thread) and a workgroup barrier per chunk.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kChains = 8;  // independent accumulators per wave in the matrix-core loops

template <int D>
__global__ void __launch_bounds__(kThreads) probe_stream_kernel(const i32x4* buf, long long run_vecs, int runs,
                                                              i32x4* out) {
  const int lane = threadIdx.x % kWave;
  const long long wid = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (wid >= runs) return;
  const i32x4* p = buf + wid * run_vecs + lane;
  const long long steps = run_vecs / kWave;  // a multiple of D (checked by the host)
  i32x4 ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) ring[u] = __builtin_nontemporal_load(p + (long long)u * kWave);
  i32x4 acc = {0, 0, 0, 0};
  for (long long s = 0; s < steps; s += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc += ring[u];
      long long n = s + u + D;
      n = n < steps ? n : steps - 1;  // the last step again past the end (not added)
      ring[u] = __builtin_nontemporal_load(p + n * kWave);
    }
  }
  out[wid * kWave + lane] = acc;
}

__global__ void __launch_bounds__(kThreads) probe_mfma_bf16_kernel(const bf16x8* ops, int iters, float* out) {
  const int lane = threadIdx.x % kWave;
  const long long wid = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    a[j] = ops[(wid * 2 * kChains + 2 * j) * kWave + lane];
    b[j] = ops[(wid * 2 * kChains + 2 * j + 1) * kWave + lane];
  }
  f32x16 acc[kChains] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[wid * kWave + lane] = s;
}

__global__ void __launch_bounds__(kThreads) probe_mfma_fp8_kernel(const i32x8* ops, int iters, float* out) {
  const int lane = threadIdx.x % kWave;
  const long long wid = (long long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  i32x8 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    a[j] = ops[(wid * 2 * kChains + 2 * j) * kWave + lane];
    b[j] = ops[(wid * 2 * kChains + 2 * j + 1) * kWave + lane];
  }
  f32x4 acc[kChains] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)  // zero scale operands: the unscaled e4m3 x e4m3 instruction
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b[j], acc[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[j][i];
  out[wid * kWave + lane] = s;
}

constexpr int kLdsThreads = 512;  // 8 waves per workgroup, two per SIMD

__global__ void __launch_bounds__(kLdsThreads) probe_lds_kernel(int iters, unsigned long long* cycles) {
  extern __shared__ i32x4 lds_buf[];  // 64 KiB used: 256 slots of 256 bytes
  for (int i = threadIdx.x; i < 4096; i += kLdsThreads) lds_buf[i] = i32x4{i, i + 1, i + 2, i + 3};
  __syncthreads();
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const unsigned long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    i32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = lds_buf[((j * 4 + lane / 16 + w * 8 + it * 3) & 255) * 16 + lane % 16];
#pragma unroll
    for (int j = 0; j < 16; ++j) asm volatile("" ::"v"(v[j]));
  }
  const unsigned long long t1 = clock64();
  if (lane == 0) cycles[blockIdx.x * (kLdsThreads / kWave) + w] = t1 - t0;
}

constexpr int kF8Slot = 272;  // the fp8 tiled GEMM's LDS slot: 16 rows x 16 bytes + padding

// NCB weight column blocks of 16 per wave: 2 with 8 waves per workgroup (two per SIMD,
// the GEMM's split), 4 with 4 waves (one per SIMD, half the LDS operand reads per
// instruction).  ops: 12 operands of 2 KiB per wave (NCB weight fragments, 8 token blocks).
template <int MODE, int NCB>
__global__ void __launch_bounds__(NCB == 2 ? 512 : 256) probe_fp8_block_kernel(const i32x8* ops, int iters, float* out,
                                                                                unsigned long long* cycles) {
  constexpr int kWaves = NCB == 2 ? 8 : 4;
  constexpr int kTbPerWave = 8 / kWaves;  // token blocks each wave initialises and stages
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // 8 x 16 slots, + staging area
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long long wid = (long long)blockIdx.x * kWaves + w;
  const i32x8* o = ops + wid * 12 * kWave + lane;
  i32x8 wf[NCB], tb[8];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) wf[cb] = o[cb * kWave];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) tb[rb] = o[(4 + rb) * kWave];
  if (MODE >= 2) {
    // every slot of this wave's token blocks gets random bytes (the wave's own operands)
    for (int q = 0; q < 16 * kTbPerWave; ++q) {
      const i32x8 v = tb[q & 7];
      *reinterpret_cast<i32x4*>(lds + (w * 16 * kTbPerWave + q) * kF8Slot + (lane % 16) * 16) =
          (lane & 16) ? i32x4{v[4], v[5], v[6], v[7]} : i32x4{v[0], v[1], v[2], v[3]};
    }
    __syncthreads();
  }
  float sa[8], wsc[NCB];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) sa[rb] = 1.0f + (float)((lane * 8 + rb) & 63) * (1.0f / 64.0f);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) wsc[cb] = 0.5f + (float)((w + cb) & 3) * 0.125f;
  f32x4 acc[8][NCB] = {};
  f32x4 p[2][NCB];
  const int rd_off = ((lane >> 4) * 2) * kF8Slot + (lane & 15) * 16;
  const unsigned long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    // the scales change from block to block in the GEMM
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) asm volatile("" : "+v"(sa[rb]));
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) asm volatile("" : "+v"(wsc[cb]));
    const int h = it & 1;
    i32x8 av[2];
    auto rd = [&](int rb) {
      if (MODE >= 2) {
        const unsigned char* ap = lds + (rb * 16 + h * 8) * kF8Slot + rd_off;
        const i32x4 l4 = *reinterpret_cast<const i32x4*>(ap);
        const i32x4 h4 = *reinterpret_cast<const i32x4*>(ap + kF8Slot);
        av[rb & 1] = i32x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
      } else {
        av[rb & 1] = tb[rb];
      }
    };
    auto fm = [&](int rb) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float sc = sa[rb] * wsc[cb];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(p[rb & 1][cb][i], sc, acc[rb][cb][i]);
      }
    };
    rd(0);
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      __builtin_amdgcn_sched_barrier(0);
      if (rb + 1 < 8) rd(rb + 1);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      if (MODE == 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[cb], av[rb & 1], acc[rb][cb], 0, 0, 0, 0, 0, 0);
          p[rb & 1][cb] = acc[rb][cb];
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          p[rb & 1][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[cb], av[rb & 1], zero, 0, 0, 0, 0, 0, 0);
        if (rb > 0) fm(rb - 1);
      }
      if (MODE == 4 && h == 1 && rb < 5) {
        // the chunk's staging writes spread over the second block's first steps
        unsigned char* st = lds + 8 * 16 * kF8Slot + w * 1024 * 5 + lane * 16;
        static_assert(MODE != 4 || NCB == 2, "spread writes with the 8-wave split only");
        if (rb < 4)
          *reinterpret_cast<i32x4*>(st + rb * 1024) = i32x4{it, rb, lane, w};
        else
          *reinterpret_cast<float*>(st + 4 * 1024) = sa[0];
      }
      if (MODE >= 2 && rb + 1 < 8) {
        if (MODE == 4 && rb < 5)
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (MODE >= 1 && rb > 0) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) asm volatile("" ::"v"(p[rb & 1][cb]));
      if (rb > 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) asm volatile("" : "+v"(acc[rb - 1][cb]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (MODE >= 1) fm(7);
    if ((MODE == 4 || MODE == 5) && h == 1) __syncthreads();
    if (MODE == 3 && h == 1) {
      // a chunk's staging writes (into an area no operand read touches) and its barrier:
      // the workgroup writes 8 x 5 KiB per chunk whatever its wave count
      unsigned char* st = lds + 8 * 16 * kF8Slot + w * 1024 * 5 * kTbPerWave + lane * 16;
#pragma unroll
      for (int i = 0; i < 4 * kTbPerWave; ++i) *reinterpret_cast<i32x4*>(st + i * 1024) = i32x4{it, i, lane, w};
#pragma unroll
      for (int i = 0; i < kTbPerWave; ++i) *reinterpret_cast<float*>(st + (4 * kTbPerWave + i) * 1024) = sa[i];
      __syncthreads();
    }
  }
  const unsigned long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s += acc[rb][cb][i];
  out[wid * kWave + lane] = s;
  if (lane == 0) cycles[wid] = t1 - t0;
}

constexpr int kBfSlot = 1056;  // the bf16 tiled GEMM's fragment slot: 1 KiB + bank padding

template <int MODE>
__global__ void __launch_bounds__(256) probe_bf16_block_kernel(const bf16x8* ops, int iters, float* out,
                                                               unsigned long long* cycles) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // 4 x 8 fragment slots + staging
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const long long wid = (long long)blockIdx.x * 4 + w;
  const bf16x8* o = ops + wid * 6 * kWave + lane;
  bf16x8 b[2], a[4];
  b[0] = o[0];
  b[1] = o[kWave];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) a[rb] = o[(2 + rb) * kWave];
  // lane l's fragment piece: row l % 32, reduction half l / 32
  const int frag_off = (lane % 32) * 16 + (lane / 32) * 528;
  if (MODE >= 1) {
    // wave w fills row block w's 8 fragment slots with its own random operand
    for (int f = 0; f < 8; ++f) *reinterpret_cast<bf16x8*>(lds + (w * 8 + f) * kBfSlot + frag_off) = a[f & 3];
    __syncthreads();
  }
  f32x16 acc[4][2] = {};
  const unsigned long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    // one 128-deep chunk: 8 fragments of 16, each feeding 4 row blocks x 2 column blocks
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      bf16x8 av[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        // the fragment order alternates between iterations, so the reads are not hoisted
        av[rb] = MODE >= 1 ? *reinterpret_cast<const bf16x8*>(lds + (rb * 8 + ((f + 4 * (it & 1)) & 7)) * kBfSlot + frag_off)
                           : a[rb];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[rb], b[cb], acc[rb][cb], 0, 0, 0);
    }
    if (MODE == 2) {
      // a chunk's staging writes (into an area no operand read touches) and its barrier
      unsigned char* st = lds + 4 * 8 * kBfSlot + w * 8 * 1024 + lane * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<i32x4*>(st + i * 1024) = i32x4{it, i, lane, w};
      __syncthreads();
    }
  }
  const unsigned long long t1 = clock64();
  float sum = 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += acc[rb][cb][i];
  out[wid * kWave + lane] = sum;
  if (lane == 0) cycles[wid] = t1 - t0;
}

}  // namespace

// buf: runs * run_bytes readable bytes (16-byte aligned); out: runs * 1 KiB.
// run_bytes must be a positive multiple of depth KiB; depth 4, 8 or 16.
// Returns 0, -1 on bad arguments, -4 on a launch error.
extern "C" int afd_probe_stream(const void* buf, long long run_bytes, int runs, int depth, void* out,
                                void* stream) {
  if (!buf || !out || runs <= 0 || run_bytes <= 0 || (run_bytes % (1024LL * depth)) != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16)
    return -1;
  const long long vecs = run_bytes / 16;
  const unsigned blocks = (unsigned)((runs + kThreads / kWave - 1) / (kThreads / kWave));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const i32x4* b = static_cast<const i32x4*>(buf);
  i32x4* o = static_cast<i32x4*>(out);
  switch (depth) {
    case 4: probe_stream_kernel<4><<<blocks, kThreads, 0, st>>>(b, vecs, runs, o); break;
    case 8: probe_stream_kernel<8><<<blocks, kThreads, 0, st>>>(b, vecs, runs, o); break;
    case 16: probe_stream_kernel<16><<<blocks, kThreads, 0, st>>>(b, vecs, runs, o); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// kind 0: bf16 (ops: waves * 16 * 1 KiB), kind 1: fp8 (ops: waves * 16 * 2 KiB);
// waves a multiple of 4; out: waves * 64 floats.  FLOPs per launch: waves * iters * 8
// * 32768 (bf16) or 65536 (fp8).
extern "C" int afd_probe_mfma(int kind, const void* ops, int waves, int iters, float* out, void* stream) {
  if (!ops || !out || waves <= 0 || waves % (kThreads / kWave) || iters <= 0 || (kind != 0 && kind != 1)) return -1;
  const unsigned blocks = (unsigned)(waves / (kThreads / kWave));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0)
    probe_mfma_bf16_kernel<<<blocks, kThreads, 0, st>>>(static_cast<const bf16x8*>(ops), iters, out);
  else
    probe_mfma_fp8_kernel<<<blocks, kThreads, 0, st>>>(static_cast<const i32x8*>(ops), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// LDS reads: `workgroups` workgroups of 8 waves, one per compute unit (96 KiB of LDS
// each), each wave reading 16 KiB per iteration; cycles: workgroups * 8 entries, each
// wave's clock64() cycles over its loop.  Returns 0, -1 on bad arguments, -4 on a launch
// error.
extern "C" int afd_probe_lds(int workgroups, int iters, unsigned long long* cycles, void* stream) {
  if (workgroups <= 0 || iters <= 0 || !cycles) return -1;
  const size_t smem = 96 * 1024;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(probe_lds_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)smem) != hipSuccess)
    return -4;
  probe_lds_kernel<<<workgroups, kLdsThreads, smem, static_cast<hipStream_t>(stream)>>>(iters, cycles);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The fp8 tiled GEMM's inner loop without global memory (mode 0 to 5, see above, with 8
// waves of 2 column blocks; modes 6 and 7: modes 2 and 3 with 4 waves of 4 column
// blocks): ops: waves * 12 * 2 KiB of random e4m3 bytes; waves a multiple of 8; out:
// waves * 64 floats; cycles: waves entries, each wave's clock64() cycles over its loop.
// FLOPs per launch: waves * iters * 16 * 65536 (modes 0-5), * 32 * 65536 (modes 6, 7).
extern "C" int afd_probe_fp8_block(int mode, const void* ops, int waves, int iters, float* out,
                                   unsigned long long* cycles, void* stream) {
  if (!ops || !out || !cycles || waves <= 0 || waves % (kLdsThreads / kWave) || iters <= 0 || mode < 0 || mode > 7)
    return -1;
  const unsigned blocks = (unsigned)(waves / (mode >= 6 ? 4 : 8));
  // 96 KiB (the loop uses 8 * 16 slots + 40 KiB of staging area): one workgroup per
  // compute unit, as the GEMM runs
  const size_t smem = 96 * 1024;
  static_assert(8 * 16 * kF8Slot + 8 * 5 * 1024 <= 96 * 1024, "the probe's LDS fits");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const i32x8* o = static_cast<const i32x8*>(ops);
  const void* fns[8] = {reinterpret_cast<const void*>(probe_fp8_block_kernel<0, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<1, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<2, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<3, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<4, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<5, 2>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<2, 4>),
                        reinterpret_cast<const void*>(probe_fp8_block_kernel<3, 4>)};
  if (hipFuncSetAttribute(fns[mode], hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess) return -4;
  switch (mode) {
    case 0: probe_fp8_block_kernel<0, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 1: probe_fp8_block_kernel<1, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 2: probe_fp8_block_kernel<2, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 3: probe_fp8_block_kernel<3, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 4: probe_fp8_block_kernel<4, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 5: probe_fp8_block_kernel<5, 2><<<blocks, 512, smem, st>>>(o, iters, out, cycles); break;
    case 6: probe_fp8_block_kernel<2, 4><<<blocks, 256, smem, st>>>(o, iters, out, cycles); break;
    default: probe_fp8_block_kernel<3, 4><<<blocks, 256, smem, st>>>(o, iters, out, cycles); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// The bf16 tiled GEMM's inner loop without global memory (mode 0, 1 or 2, see above):
// ops: waves * 6 KiB of random bf16 bytes; waves a multiple of 4; out: waves * 64 floats;
// cycles: waves entries, each wave's clock64() cycles over its loop.  FLOPs per launch:
// waves * iters * 64 * 32768.
extern "C" int afd_probe_bf16_block(int mode, const void* ops, int waves, int iters, float* out,
                                    unsigned long long* cycles, void* stream) {
  if (!ops || !out || !cycles || waves <= 0 || waves % 4 || iters <= 0 || mode < 0 || mode > 2) return -1;
  const unsigned blocks = (unsigned)(waves / 4);
  // 96 KiB: one workgroup per compute unit, as the GEMM runs
  const size_t smem = 96 * 1024;
  static_assert(4 * 8 * kBfSlot + 4 * 8 * 1024 <= 96 * 1024, "the probe's LDS fits");
  const void* fns[3] = {reinterpret_cast<const void*>(probe_bf16_block_kernel<0>),
                        reinterpret_cast<const void*>(probe_bf16_block_kernel<1>),
                        reinterpret_cast<const void*>(probe_bf16_block_kernel<2>)};
  if (hipFuncSetAttribute(fns[mode], hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess) return -4;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bf16x8* o = static_cast<const bf16x8*>(ops);
  switch (mode) {
    case 0: probe_bf16_block_kernel<0><<<blocks, 256, smem, st>>>(o, iters, out, cycles); break;
    case 1: probe_bf16_block_kernel<1><<<blocks, 256, smem, st>>>(o, iters, out, cycles); break;
    default: probe_bf16_block_kernel<2><<<blocks, 256, smem, st>>>(o, iters, out, cycles); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
