// Weighted combine back to token order: y[t] = sum_j gate[t, j] * O[pos(t, j)], in
// slot order with fp32 accumulation and one final rounding, plus the shared
// expert's output with gate 1 ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §3: the FFN service returns the layer output of every token it received).
// Grid: (token, 1024-channel chunk) for small batches, so even a decode batch of a
// few tokens spreads over many workgroups; one workgroup per token that walks its
// channels for large batches.  A thread handles 4 consecutive channels at a time.
// The k rows of a channel group are all loaded before they are summed (KU = k
// rounded up to 8 or 32, the loop fully unrolled); the sum itself stays in slot
// order.  Large batches read the rows nontemporally (each is read once); decode
// batches use plain loads, their rows being still in L2 from the down projection.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxK = 32;

template <bool NT>
__device__ __forceinline__ float4 load_row4(const float* p) {
  if (NT) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  return *reinterpret_cast<const float4*>(p);
}

template <bool BF16_OUT, int KU, bool NT>
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
  for (int c = blockIdx.y * kCombineThreads + threadIdx.x; c < H / 4; c += gridDim.y * kCombineThreads) {
  float4 o[KU];
#pragma unroll
  for (int j = 0; j < KU; ++j)
    if (j < k) o[j] = load_row4<NT>(O + (size_t)pos_s[j] * H + 4 * c);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KU; ++j) {
    if (j < k) {
      const float gj = g_s[j];
      acc.x = fmaf(gj, o[j].x, acc.x);
      acc.y = fmaf(gj, o[j].y, acc.y);
      acc.z = fmaf(gj, o[j].z, acc.z);
      acc.w = fmaf(gj, o[j].w, acc.w);
    }
  }
  if (Os) {
    const float4 v = load_row4<NT>(Os + (size_t)t * H + 4 * c);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
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

template <bool BF16_OUT, bool NT>
static void launch_combine_t(dim3 grid, const float* O, const float* Os, const float* gates, const int32_t* pair_pos,
                             int k, int H, void* y, hipStream_t st) {
  if (k <= 8)
    combine_kernel<BF16_OUT, 8, NT><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  else
    combine_kernel<BF16_OUT, kCombineMaxK, NT><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
}

hipError_t launch_combine(const float* O, const float* Os, const float* gates, const int32_t* pair_pos, int T, int k,
                          int H, void* y, bool y_bf16, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (k > kCombineMaxK || H % 4) return hipErrorInvalidValue;
  // small batches split each token's channels over workgroups; large ones give each
  // token one workgroup that walks its channels
  const int chunks = (H / 4 + kCombineThreads - 1) / kCombineThreads;
  const dim3 grid((unsigned)T, (unsigned)(T >= 8192 ? 1 : chunks));
  // rows far beyond the L2 capacity are read nontemporally
  const bool nt = (long long)T * k * H * 4 > (256ll << 20);
  if (y_bf16) {
    if (nt)
      launch_combine_t<true, true>(grid, O, Os, gates, pair_pos, k, H, y, st);
    else
      launch_combine_t<true, false>(grid, O, Os, gates, pair_pos, k, H, y, st);
  } else {
    if (nt)
      launch_combine_t<false, true>(grid, O, Os, gates, pair_pos, k, H, y, st);
    else
      launch_combine_t<false, false>(grid, O, Os, gates, pair_pos, k, H, y, st);
  }
  return hipGetLastError();
}

}  // namespace afd
