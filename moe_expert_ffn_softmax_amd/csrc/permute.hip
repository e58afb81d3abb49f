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
#include "route.h"

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

// The whole sort in one workgroup of kPermuteThreads threads; `ids` may point to
// global memory or to LDS.
__device__ __forceinline__ void permute_one_workgroup(const int32_t* ids, int P, int E, int32_t* __restrict__ counts,
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

__global__ void __launch_bounds__(kPermuteThreads) permute_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_pair,
                                                                  int32_t* __restrict__ pair_pos) {
  permute_one_workgroup(ids, P, E, counts, offsets, sorted_pair, pair_pos);
}

// Decode batches (at most kRouteSmallTokens tokens): routing and the sort in one
// workgroup, so the route call is a single launch.  Wave w routes tokens w, w + 16,
// ...; the experts go to LDS as well as to ids, and the sort reads them from there.
constexpr int kRouteSmallTokens = 64;

template <int PER_LANE>
__global__ void __launch_bounds__(kPermuteThreads) route_small_kernel(const float* __restrict__ logits,
                                                                      const float* __restrict__ sel_bias, int T, int E,
                                                                      int k, int32_t* __restrict__ ids,
                                                                      float* __restrict__ gates,
                                                                      int32_t* __restrict__ counts,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ sorted_pair,
                                                                      int32_t* __restrict__ pair_pos) {
  __shared__ int32_t ids_s[kRouteSmallTokens * kRouterMaxSlots];
  const int lane = lane_id();
  for (int t = threadIdx.x / kWave; t < T; t += kPermuteWaves) {
    int id;
    float gate;
    route_token<PER_LANE>(logits + (size_t)t * E, sel_bias, E, k, &id, &gate);
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      gates[(size_t)t * k + lane] = gate;
      ids_s[t * k + lane] = id;
    }
  }
  __syncthreads();
  permute_one_workgroup(ids_s, T * k, E, counts, offsets, sorted_pair, pair_pos);
}

hipError_t launch_route_small(const float* logits, const float* sel_bias, int T, int E, int k, int32_t* ids,
                              float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                              int32_t* pair_pos, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (T > kRouteSmallTokens || k > kRouterMaxSlots || E > kPermuteMaxE) return hipErrorInvalidValue;
#define AFD_ROUTE_SMALL(PL) \
  route_small_kernel<PL><<<1, kPermuteThreads, 0, st>>>(logits, sel_bias, T, E, k, ids, gates, counts, offsets, sorted_pair, pair_pos)
  if (E <= 64)
    AFD_ROUTE_SMALL(1);
  else if (E <= 128)
    AFD_ROUTE_SMALL(2);
  else if (E <= 256)
    AFD_ROUTE_SMALL(4);
  else if (E <= 512)
    AFD_ROUTE_SMALL(8);
  else
    AFD_ROUTE_SMALL(kRouterMaxPerLane);
#undef AFD_ROUTE_SMALL
  return hipGetLastError();
}

int route_small_tokens() { return kRouteSmallTokens; }

// ---------------------------------------------------------------------------------
// Large batches: the same three steps spread over blocks of kPermuteBlock pairs.
//   histogram  (blocks 0 .. NB-2): block b counts its pairs per expert and leaves the
//              counts in pair_pos[b*kPermuteBlock + e] (inside its own pair range);
//   scan       (one workgroup): per expert, running sums over the blocks replace those
//              counts (block bases without the expert offset); the last block's pairs
//              are counted here; totals give counts and the offsets;
//   scatter    (all blocks): block b reads its bases back from its own range, then
//              places its pairs as the one-workgroup kernel does, which overwrites
//              that range with the final pair positions.  The last block's bases are
//              offsets[e + 1] minus its own counts.
// Only block b ever reads or writes pair_pos inside its own range, and the reads come
// before a barrier that precedes the writes, so the staging needs no extra memory.
constexpr int kPermuteBlock = 4096;  // pairs per block (>= E, which is at most 1024)

// Per-wave expert counts of the pairs [begin, end) split into 16 contiguous wave
// chunks (multiples of 64): base[w][e] += count.  base must be zeroed.  Returns the
// wave's chunk through *wb, *we.
__device__ __forceinline__ void wave_chunk_histogram(const int32_t* __restrict__ ids, int begin, int end, int nbits,
                                                     int (*base)[kPermuteMaxE], int* wb, int* we) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int n = end - begin;
  const int per_wave = ((n + kPermuteWaves - 1) / kPermuteWaves + kWave - 1) / kWave * kWave;
  const int b = min(end, begin + w * per_wave);
  const int e = min(end, b + per_wave);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int p0 = b; p0 < e; p0 += kWave) {
    const int p = p0 + lane;
    const bool ok = p < e;
    const int id = ok ? ids[p] : 0;
    const uint64_t m = match_lanes(id, nbits, __ballot(ok));
    if (ok && (m & lt_mask) == 0) base[w][id] += __popcll(m);
  }
  *wb = b;
  *we = e;
}

__device__ __forceinline__ int expert_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

__global__ void __launch_bounds__(kPermuteThreads) permute_hist_kernel(const int32_t* __restrict__ ids, int E,
                                                                       int32_t* __restrict__ pair_pos) {
  __shared__ int base[kPermuteWaves][kPermuteMaxE];
  for (int i = threadIdx.x; i < kPermuteWaves * E; i += kPermuteThreads) base[i / E][i % E] = 0;
  __syncthreads();
  const int begin = blockIdx.x * kPermuteBlock;
  int wb, we;
  wave_chunk_histogram(ids, begin, begin + kPermuteBlock, expert_bits(E), base, &wb, &we);
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    int c = 0;
    for (int v = 0; v < kPermuteWaves; ++v) c += base[v][e];
    pair_pos[begin + e] = c;
  }
}

__global__ void __launch_bounds__(kPermuteThreads) permute_scan_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                       int nb, int32_t* __restrict__ counts,
                                                                       int32_t* __restrict__ offsets,
                                                                       int32_t* __restrict__ pair_pos) {
  __shared__ int base[kPermuteWaves][kPermuteMaxE];
  __shared__ int scan_tmp[kPermuteWaves + 1];
  for (int i = threadIdx.x; i < kPermuteWaves * E; i += kPermuteThreads) base[i / E][i % E] = 0;
  __syncthreads();
  int wb, we;
  wave_chunk_histogram(ids, (nb - 1) * kPermuteBlock, P, expert_bits(E), base, &wb, &we);
  __syncthreads();
  const int e = threadIdx.x;
  int total_e = 0;
  if (e < E) {
    for (int b = 0; b < nb - 1; ++b) {
      int32_t* slot = pair_pos + (size_t)b * kPermuteBlock + e;
      const int c = *slot;
      *slot = total_e;
      total_e += c;
    }
    for (int v = 0; v < kPermuteWaves; ++v) total_e += base[v][e];
    counts[e] = total_e;
  }
  int total = 0;
  const int excl = block_exclusive_scan(e < E ? total_e : 0, scan_tmp, &total);
  if (e < E) offsets[e] = excl;
  if (e == 0) offsets[E] = total;
}

__global__ void __launch_bounds__(kPermuteThreads) permute_scatter_kernel(const int32_t* __restrict__ ids, int P,
                                                                          int E, int nb,
                                                                          const int32_t* __restrict__ offsets,
                                                                          int32_t* __restrict__ sorted_pair,
                                                                          int32_t* __restrict__ pair_pos) {
  __shared__ int base[kPermuteWaves][kPermuteMaxE];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int nbits = expert_bits(E);
  const bool last = blockIdx.x == nb - 1;
  const int begin = blockIdx.x * kPermuteBlock;
  const int end = min(P, begin + kPermuteBlock);
  for (int i = threadIdx.x; i < kPermuteWaves * E; i += kPermuteThreads) base[i / E][i % E] = 0;
  // this block's bases (before the barrier that precedes every write of pair_pos)
  const int e = threadIdx.x;
  int blk = 0;
  if (e < E) blk = last ? 0 : pair_pos[begin + e] + offsets[e];
  __syncthreads();
  int wb, we;
  wave_chunk_histogram(ids, begin, end, nbits, base, &wb, &we);
  __syncthreads();
  if (e < E) {
    int run = 0;
    for (int v = 0; v < kPermuteWaves; ++v) run += base[v][e];
    // the last block ends exactly at the end of each expert's segment
    int b0 = last ? offsets[e + 1] - run : blk;
    for (int v = 0; v < kPermuteWaves; ++v) {
      const int c = base[v][e];
      base[v][e] = b0;
      b0 += c;
    }
  }
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int p0 = wb; p0 < we; p0 += kWave) {
    const int p = p0 + lane;
    const bool ok = p < we;
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
  if (E > kPermuteMaxE || E > kPermuteBlock) return hipErrorInvalidValue;
  if (P <= 2 * kPermuteBlock) {
    permute_kernel<<<1, kPermuteThreads, 0, st>>>(ids, P, E, counts, offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  const int nb = (P + kPermuteBlock - 1) / kPermuteBlock;
  if (nb > 1) permute_hist_kernel<<<nb - 1, kPermuteThreads, 0, st>>>(ids, E, pair_pos);
  permute_scan_kernel<<<1, kPermuteThreads, 0, st>>>(ids, P, E, nb, counts, offsets, pair_pos);
  permute_scatter_kernel<<<nb, kPermuteThreads, 0, st>>>(ids, P, E, nb, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace afd
