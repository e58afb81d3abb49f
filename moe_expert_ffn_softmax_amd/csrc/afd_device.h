// Device-side helpers shared by the gfx950 kernels of the expert-FFN layer:
// vector types for the matrix-core operands, bf16 conversions, wave64 reductions
// and a block-wide exclusive scan.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afd {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float f) { return static_cast<__bf16>(f); }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }

// e4m3 codes of four values already divided by their scale, |v| clamped to 448
// (values between 448 and the next binade would otherwise leave the e4m3 range);
// the hardware conversion rounds to nearest even.  Byte i holds value i.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// SiLU(z) = z * sigmoid(z).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (l >= off) v += o;
  }
  return v;
}

// Exclusive scan over one int per thread of the block (blockDim.x <= 1024).
// `smem` needs blockDim.x / 64 + 1 ints.  Returns the thread's exclusive prefix and
// writes the block total to *total.  Contains __syncthreads().
__device__ __forceinline__ int block_exclusive_scan(int v, int* smem, int* total) {
  const int l = lane_id();
  const int w = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_inclusive_scan(v);
  if (l == kWave - 1) smem[w] = inc;
  __syncthreads();
  if (w == 0) {
    int s = l < nw ? smem[l] : 0;
    int si = wave_inclusive_scan(s);
    if (l < nw) smem[l] = si - s;
    if (l == nw - 1) smem[nw] = si;
  }
  __syncthreads();
  int r = inc - v + smem[w];
  *total = smem[nw];
  __syncthreads();
  return r;
}

}  // namespace afd
