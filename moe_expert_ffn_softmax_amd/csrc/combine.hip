// Weighted combine back to token order: y[t] = sum_j gate[t, j] * O[pos(t, j)], in
// slot order with fp32 accumulation and one final rounding, plus the shared
// expert's output with gate 1 ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §3: the FFN service returns the layer output of every token it received).
// One workgroup per token; each thread handles 4 consecutive channels.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxK = 32;

template <bool BF16_OUT>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const float* __restrict__ O,
                                                                  const float* __restrict__ Os,
                                                                  const float* __restrict__ gates,
                                                                  const int32_t* __restrict__ pair_pos, int k, int H,
                                                                  void* __restrict__ y) {
  __shared__ float g_s[kCombineMaxK];
  __shared__ int pos_s[kCombineMaxK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    g_s[threadIdx.x] = gates[(size_t)t * k + threadIdx.x];
    pos_s[threadIdx.x] = pair_pos[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int H4 = H / 4;
  for (int c = threadIdx.x; c < H4; c += kCombineThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 o = reinterpret_cast<const float4*>(O + (size_t)pos_s[j] * H)[c];
      const float gj = g_s[j];
      acc.x = fmaf(gj, o.x, acc.x);
      acc.y = fmaf(gj, o.y, acc.y);
      acc.z = fmaf(gj, o.z, acc.z);
      acc.w = fmaf(gj, o.w, acc.w);
    }
    if (Os) {
      const float4 o = reinterpret_cast<const float4*>(Os + (size_t)t * H)[c];
      acc.x += o.x;
      acc.y += o.y;
      acc.z += o.z;
      acc.w += o.w;
    }
    if (BF16_OUT) {
      uint2 pk;
      pk.x = (uint32_t)bf16_bits(f32_to_bf16(acc.x)) | ((uint32_t)bf16_bits(f32_to_bf16(acc.y)) << 16);
      pk.y = (uint32_t)bf16_bits(f32_to_bf16(acc.z)) | ((uint32_t)bf16_bits(f32_to_bf16(acc.w)) << 16);
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (size_t)t * H)[c] = pk;
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * H)[c] = acc;
    }
  }
}

hipError_t launch_combine(const float* O, const float* Os, const float* gates, const int32_t* pair_pos, int T, int k,
                          int H, void* y, bool y_bf16, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (k > kCombineMaxK || H % 4) return hipErrorInvalidValue;
  if (y_bf16)
    combine_kernel<true><<<T, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  else
    combine_kernel<false><<<T, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  return hipGetLastError();
}

}  // namespace afd
