// Per-token top-k selection shared by the router kernel and the fused decode-batch
// route kernel (see router.hip for the method and its source).
#pragma once
#include "afd_device.h"

namespace afd {

constexpr int kRouterMaxPerLane = 16;  // E <= 1024
constexpr int kRouterMaxSlots = 32;    // k <= 32

__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float unordered_bits(uint32_t o) {
  uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Route one token with one wave: lane j < k returns the expert of slot j in *id and
// its gate in *gate (other lanes: unspecified).
//
// sel_bias == NULL: the experts are ranked on the logits themselves and the gates are
// the softmax of the selected logits.  sel_bias != NULL (a per-expert bias that only
// steers the choice, the dynamic-bias load balancing of "MoE 大规模分布式推理工程实战：
// 从 All-to-All 通信到动态专家放置", §4.1, in its selection-only form): the experts are
// ranked on the fp32 sum row[e] + sel_bias[e], and the gates are the softmax of the
// unbiased row values of the chosen experts, renormalised over them.
template <int PER_LANE>
__device__ __forceinline__ void route_token(const float* __restrict__ row, const float* __restrict__ sel_bias,
                                            int E, int k, int* id, float* gate) {
  const int lane = lane_id();
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + i * kWave;
    float v = 0.0f;
    if (e < E) v = sel_bias ? row[e] + sel_bias[e] : row[e];
    key[i] = e < E ? ((uint64_t)ordered_bits(v) << 32) | (uint32_t)(~(uint32_t)e) : 0ull;
  }
  float sel_val = 0.0f;  // lane j keeps the logit of slot j
  int sel_id = 0;
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    const float v = unordered_bits((uint32_t)(best >> 32));
    if (j == 0) top = v;
    if (lane == j) {
      sel_val = v;
      sel_id = e;
    }
    if ((e & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (i == e / kWave) key[i] = 0;
    }
  }
  if (sel_bias) {
    // the keys held score + bias: take the chosen experts' unbiased scores instead
    sel_val = lane < k ? row[sel_id] : -INFINITY;
    top = wave_max_f32(sel_val);
  }
  const float ex = lane < k ? expf(sel_val - top) : 0.0f;
  const float sum = wave_sum_f32(ex);
  *id = sel_id;
  *gate = ex / sum;
}

}  // namespace afd
