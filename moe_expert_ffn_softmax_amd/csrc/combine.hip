// Weighted combine back to token order: y[t] = sum_j gate[t, j] * O[pos(t, j)], in
// slot order with fp32 accumulation and one final rounding, plus the shared
// expert's output with gate 1 ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
// §3: the FFN service returns the layer output of every token it received).
// The rows O and Os are in the layer's activation type (bf16 for the bf16 and fp8
// layers, fp32 for the fp32 layer), and so is y.
// Grid: (token, channel chunk) for small batches, so even a decode batch of a few
// tokens spreads over many workgroups; one workgroup per token that walks its
// channels for large batches.  A thread handles 16 bytes of each row at a time (8
// bf16 or 4 fp32 channels).  The k rows of a channel group are all loaded before
// they are summed (KU = k rounded up to 8 or 32, the loop fully unrolled); the sum
// itself stays in slot order.  Large batches read the rows nontemporally (each is
// read once); decode batches use plain loads, their rows being still in L2 from the
// down projection.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kCombineThreads = 256;
constexpr int kCombineMaxK = 32;

template <bool NT>
__device__ __forceinline__ i32x4 load16(const char* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
  return *reinterpret_cast<const i32x4*>(p);
}

// The V = 8 (bf16) or 4 (fp32) channels held in 16 bytes, as fp32.
template <bool BF16>
__device__ __forceinline__ void unpack16(const i32x4 r, float* v) {
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(static_cast<uint32_t>(r[i]) << 16);
      v[2 * i + 1] = __uint_as_float(static_cast<uint32_t>(r[i]) & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __int_as_float(r[i]);
  }
}

template <bool BF16, int KU, bool NT, bool APPLY = true>
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const void* __restrict__ O,
                                                                  const void* __restrict__ Os,
                                                                  const float* __restrict__ gates,
                                                                  const int32_t* __restrict__ pair_pos, int k, int H,
                                                                  void* __restrict__ y) {
  constexpr int V = BF16 ? 8 : 4;
  constexpr int kElt = BF16 ? 2 : 4;
  __shared__ float g_s[kCombineMaxK];
  __shared__ int pos_s[kCombineMaxK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    g_s[threadIdx.x] = gates[(size_t)t * k + threadIdx.x];
    pos_s[threadIdx.x] = pair_pos[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const size_t row_bytes = (size_t)H * kElt;
  for (int c = blockIdx.y * kCombineThreads + threadIdx.x; c < H / V; c += gridDim.y * kCombineThreads) {
    i32x4 raw[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j)  // a slot with gate 0 adds nothing and is not read
      if (j < k && g_s[j] != 0.f)
        raw[j] = load16<NT>(static_cast<const char*>(O) + (size_t)pos_s[j] * row_bytes + 16 * (size_t)c);
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      if (j < k && g_s[j] != 0.f) {
        const float gj = g_s[j];
        float v[V];
        unpack16<BF16>(raw[j], v);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = APPLY ? fmaf(gj, v[i], acc[i]) : acc[i] + v[i];
      }
    }
    if (Os) {
      float v[V];
      unpack16<BF16>(load16<NT>(static_cast<const char*>(Os) + (size_t)t * row_bytes + 16 * (size_t)c), v);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    i32x4 out;
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[i] = (int)((uint32_t)bf16_bits(f32_to_bf16(acc[2 * i])) |
                       ((uint32_t)bf16_bits(f32_to_bf16(acc[2 * i + 1])) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = __float_as_int(acc[i]);
    }
    *reinterpret_cast<i32x4*>(static_cast<char*>(y) + (size_t)t * row_bytes + 16 * (size_t)c) = out;
  }
}

template <bool BF16, bool NT>
static void launch_combine_t(dim3 grid, const void* O, const void* Os, const float* gates, const int32_t* pair_pos,
                             int k, int H, void* y, hipStream_t st, bool applied) {
  if (applied) {  // the fused decode launch's rows (bf16, decode batches: k <= 32, plain loads)
    if (k <= 8)
      combine_kernel<BF16, 8, NT, false><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
    else
      combine_kernel<BF16, kCombineMaxK, NT, false><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  } else if (k <= 8) {
    combine_kernel<BF16, 8, NT><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  } else {
    combine_kernel<BF16, kCombineMaxK, NT><<<grid, kCombineThreads, 0, st>>>(O, Os, gates, pair_pos, k, H, y);
  }
}

hipError_t launch_combine(const void* O, const void* Os, const float* gates, const int32_t* pair_pos, int T, int k,
                          int H, void* y, bool bf16, hipStream_t st, bool gates_applied) {
  if (T <= 0) return hipSuccess;
  const int v = bf16 ? 8 : 4;
  if (k > kCombineMaxK || H % v) return hipErrorInvalidValue;
  // small batches split each token's channels over workgroups; large ones give each
  // token one workgroup that walks its channels
  const int chunks = (H / v + kCombineThreads - 1) / kCombineThreads;
  const dim3 grid((unsigned)T, (unsigned)(T >= 8192 ? 1 : chunks));
  // rows far beyond the L2 capacity are read nontemporally
  const bool nt = (long long)T * k * H * (bf16 ? 2 : 4) > (256ll << 20);
  if (bf16) {
    if (nt)
      launch_combine_t<true, true>(grid, O, Os, gates, pair_pos, k, H, y, st, gates_applied);
    else
      launch_combine_t<true, false>(grid, O, Os, gates, pair_pos, k, H, y, st, gates_applied);
  } else {
    if (nt)
      launch_combine_t<false, true>(grid, O, Os, gates, pair_pos, k, H, y, st, gates_applied);
    else
      launch_combine_t<false, false>(grid, O, Os, gates, pair_pos, k, H, y, st, gates_applied);
  }
  return hipGetLastError();
}

}  // namespace afd
