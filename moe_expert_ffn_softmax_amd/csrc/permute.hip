// Token-to-expert permute: a stable counting sort of the P = T*k (token, slot) pairs
// by expert, in one workgroup.
//
// The steps are those of the count / prefix-sum / pack sequence of "MoE 大规模分布式
// 推理工程实战：从 All-to-All 通信到动态专家放置", §2.2, applied per expert instead of
// per destination GPU (and the pre-sorting of routed tokens recommended by the
// omica.com.cn AFD article, §3.3):
//   1. histogram: each of the 16 waves counts the experts of its contiguous chunk
//      of pairs;
//   2. scan: per expert, the wave counts are turned into running bases; their totals
//      are the expert counts, whose exclusive block scan gives the offsets;
//   3. scatter: each wave walks its chunk again in ascending pair order and places
//      every pair at its expert's base plus its rank.
// Within 64 consecutive pairs the lanes holding the same expert are found with
// ceil(log2 E) ballots over the bits of the expert id (no atomics), so ranks come
// out in ascending pair order and the result is deterministic: inside an expert's
// segment pairs are ordered by token.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteWaves = kPermuteThreads / kWave;
constexpr int kPermuteMaxE = 1024;

// Lanes (among `valid`) whose expert id equals this lane's.
__device__ __forceinline__ uint64_t match_lanes(int id, int nbits, uint64_t valid) {
  uint64_t m = valid;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (id >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__global__ void __launch_bounds__(kPermuteThreads) permute_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_pair,
                                                                  int32_t* __restrict__ pair_pos) {
  __shared__ int base[kPermuteWaves][kPermuteMaxE];
  __shared__ int scan_tmp[kPermuteWaves + 1];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  for (int i = threadIdx.x; i < kPermuteWaves * E; i += kPermuteThreads) base[i / E][i % E] = 0;
  __syncthreads();

  // contiguous chunk of this wave, a multiple of 64 pairs
  const int per_wave = ((P + kPermuteWaves - 1) / kPermuteWaves + kWave - 1) / kWave * kWave;
  const int begin = min(P, w * per_wave);
  const int end = min(P, begin + per_wave);
  const uint64_t lt_mask = (1ull << lane) - 1ull;

  // 1. histogram of the chunk
  for (int p0 = begin; p0 < end; p0 += kWave) {
    const int p = p0 + lane;
    const bool ok = p < end;
    const int id = ok ? ids[p] : 0;
    const uint64_t m = match_lanes(id, nbits, __ballot(ok));
    if (ok && (m & lt_mask) == 0) base[w][id] += __popcll(m);
  }
  __syncthreads();

  // 2. per-expert running bases over the waves, counts, exclusive scan -> offsets
  const int e = threadIdx.x;  // E <= 1024 = blockDim.x
  int total_e = 0;
  if (e < E) {
    for (int v = 0; v < kPermuteWaves; ++v) {
      const int c = base[v][e];
      base[v][e] = total_e;
      total_e += c;
    }
    counts[e] = total_e;
  }
  int total = 0;
  const int excl = block_exclusive_scan(e < E ? total_e : 0, scan_tmp, &total);
  if (e < E) {
    offsets[e] = excl;
    for (int v = 0; v < kPermuteWaves; ++v) base[v][e] += excl;
  }
  if (e == 0) offsets[E] = total;
  __syncthreads();

  // 3. scatter in ascending pair order
  for (int p0 = begin; p0 < end; p0 += kWave) {
    const int p = p0 + lane;
    const bool ok = p < end;
    const int id = ok ? ids[p] : 0;
    const uint64_t m = match_lanes(id, nbits, __ballot(ok));
    int pos = 0;
    if (ok) pos = base[w][id] + __popcll(m & lt_mask);
    __builtin_amdgcn_wave_barrier();
    if (ok && (m & lt_mask) == 0) base[w][id] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
  }
}

hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, hipStream_t st) {
  if (E > kPermuteMaxE) return hipErrorInvalidValue;
  permute_kernel<<<1, kPermuteThreads, 0, st>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace afd
