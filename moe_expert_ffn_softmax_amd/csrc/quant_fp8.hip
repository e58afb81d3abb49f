// Activation quantisation to fp8 (OCP e4m3) per row and per 128 channels, for the
// fp8 layer: scale = amax / 448 (1 for an all-zero group), code = nearest e4m3 of
// v / scale, ties to even, both divisions IEEE fp32.  The weights of that layer carry
// one fp32 scale per 128x128 block; the activations (x before the gate/up projection
// and h before the down projection) get one per row per 128 channels, so every
// 128-deep block of a product has one scale on each side.  FP8/BF16 mixed precision
// is the omica.com.cn AFD article's §3.3 ("FP8BF16混合精度").
//
// One wave per (row, 2 groups): lane l handles 4 consecutive channels of group
// (l / 32); the group amax is a 32-lane max.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ float load_act(const void* p, size_t i, bool bf16) {
  if (bf16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

// rows x cols activations (bf16 or fp32, row stride ld) -> codes [rows, cols] and
// scales [rows, cols / 128].  `row_index` (optional) gathers source rows.
__global__ void __launch_bounds__(kQuantThreads) quant_fp8_kernel(const void* __restrict__ src, int rows, int cols,
                                                                  int ld, bool src_bf16, uint8_t* __restrict__ q,
                                                                  float* __restrict__ scales) {
  const int lane = lane_id();
  const int groups = cols / 128;
  const int pairs = (groups + 1) / 2;
  const long long wave = (long long)blockIdx.x * (kQuantThreads / kWave) + threadIdx.x / kWave;
  const long long waves = (long long)gridDim.x * (kQuantThreads / kWave);
  for (long long wi = wave; wi < (long long)rows * pairs; wi += waves) {
    const int r = (int)(wi / pairs);
    const int g = (int)(wi % pairs) * 2 + lane / 32;
    const bool ok = g < groups;
    const int c0 = g * 128 + (lane & 31) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = load_act(src, (size_t)r * ld + c0 + i, src_bf16);
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    if (ok) {
      const uint32_t pk = e4m3_pack4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
      *reinterpret_cast<uint32_t*>(q + (size_t)r * cols + c0) = pk;
      if ((lane & 31) == 0) scales[(size_t)r * groups + g] = s;
    }
  }
}

hipError_t launch_quant_fp8(const void* src, int rows, int cols, int ld, bool src_bf16, uint8_t* q, float* scales,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (cols % 128) return hipErrorInvalidValue;
  const long long work = (long long)rows * ((cols / 128 + 1) / 2);
  long long blocks = (work + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  quant_fp8_kernel<<<(unsigned)blocks, kQuantThreads, 0, st>>>(src, rows, cols, ld, src_bf16, q, scales);
  return hipGetLastError();
}

}  // namespace afd
