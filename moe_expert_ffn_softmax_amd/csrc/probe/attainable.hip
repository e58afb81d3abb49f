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
