// Top-k softmax router: one wave64 per token.
//
// Selects, per token, the k experts with the largest fp32 logits (ties to the lower
// expert index) and gates = their softmax probabilities renormalised over the k
// (the router of "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家放置",
// §4.1: top-k of the logits, then a softmax over the selected ones).  The softmax
// denominator over all E cancels in the renormalisation, so the gate of slot j is
// exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected experts, l_0 the largest.
//
// Selection compares raw fp32 logits through an order-preserving 64-bit key:
// high word = the float's bits mapped to unsigned order (-0 folded onto +0, so the
// two compare equal as in IEEE), low word = ~expert, so the larger key is the larger
// logit and, on a tie, the lower expert.  k rounds of a wave-wide max pick the
// experts in slot order; the lane that owns the winner retires it.  With a
// selection-only bias the keys are built from logit + bias (see route.h).
#include "afd_device.h"
#include "afd_internal.h"
#include "route.h"

namespace afd {

template <int PER_LANE>
__global__ void __launch_bounds__(256) router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ sel_bias, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int id;
  float gate;
  route_token<PER_LANE>(logits + (size_t)t * E, sel_bias, E, k, &id, &gate);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    gates[(size_t)t * k + lane] = gate;
  }
}

hipError_t launch_router(const float* logits, const float* sel_bias, int T, int E, int k, int32_t* ids, float* gates,
                         hipStream_t st) {
  if (T <= 0) return hipSuccess;
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
  if (E <= 64)
    router_topk_kernel<1><<<grid, block, 0, st>>>(logits, sel_bias, T, E, k, ids, gates);
  else if (E <= 128)
    router_topk_kernel<2><<<grid, block, 0, st>>>(logits, sel_bias, T, E, k, ids, gates);
  else if (E <= 256)
    router_topk_kernel<4><<<grid, block, 0, st>>>(logits, sel_bias, T, E, k, ids, gates);
  else if (E <= 512)
    router_topk_kernel<8><<<grid, block, 0, st>>>(logits, sel_bias, T, E, k, ids, gates);
  else
    router_topk_kernel<kRouterMaxPerLane><<<grid, block, 0, st>>>(logits, sel_bias, T, E, k, ids, gates);
  return hipGetLastError();
}

}  // namespace afd
