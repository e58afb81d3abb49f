// Capacity-aware routing: the adaptive token dropper of "MoE 大规模分布式推理工程实战：从
// All-to-All 通信到动态专家放置", §4.2.
//
// Per batch the per-expert counts start at zero.  Tokens are decided in order: a token
// goes to the first expert of its preference list whose count is under its limit (with
// that slot's gate) and to no other; when all are full, the least-loaded expert (lowest
// index on ties) takes it at half the first gate if its count is under 1.5x its limit;
// otherwise it is dropped.  Afterwards the limits adapt: x1.2 (truncated) when reached,
// x0.9 (truncated, not below the base) when under half used.
//
// Each decision depends on every earlier one, so one workgroup does the walk.  Wave 0
// decides 64 tokens at a time: each lane finds its token's first preference with room
// under the counts at the chunk's start, and the chunk commits in one step up to the
// first lane whose choice those counts cannot vouch for: an expert that fills inside the
// chunk (the next chunk starts at that token), or a token whose every preference is full
// (it is decided alone with the least-loaded rule, and the next chunk starts after it).
// A batch with room everywhere costs T/64 chunks; each expert filling up and each
// fallback or drop adds one.  A lane's rank among the chunk's lanes choosing the same
// expert comes from ten ballots over the expert id's bits, so it is also the token's
// place in that expert's list; it rides in the upper bits of assign until the offsets
// are known, and a last parallel pass places the tokens.  Counts, limits and the staged
// preference lists live in LDS; the limit products are exact integer forms of the
// truncated scalings (6L/5 and 9L/10, 2c < 3L for c < 1.5L, 2c < L for c < L/2).
#include <limits.h>

#include "capacity.h"

namespace afd {
namespace {

constexpr int kCapThreads = 256;      // four waves stage the lists; wave 0 decides
constexpr int kCapMaxE = 1024;
constexpr int kCapStageSlots = 4096;  // preference slots (tokens * k) staged per pass

__device__ __forceinline__ unsigned long long lanes_below(int lane) { return (1ull << lane) - 1ull; }

constexpr int kPosShift = 10;  // assign holds expert | place << 10 until the last pass

// First slot of staged token i whose expert is under its limit: the expert, with *slot
// and *cnt (its count) set, or -1.  Eight slots are tested per step so their LDS reads
// overlap.
__device__ __forceinline__ int first_with_room(const int32_t* s_ids, const int32_t* s_cnt, const int32_t* s_lim,
                                               int i, int k, int E, int* slot, int* cnt, int* lim) {
  for (int j0 = 0; j0 < k; j0 += 8) {
    int e[8], c[8], l[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) e[u] = j0 + u < k ? s_ids[i * k + j0 + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ec = (unsigned)e[u] < (unsigned)E ? e[u] : 0;
      c[u] = s_cnt[ec];
      l[u] = s_lim[ec];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if ((unsigned)e[u] < (unsigned)E && c[u] < l[u]) {
        *slot = j0 + u;
        *cnt = c[u];
        *lim = l[u];
        return e[u];
      }
  }
  return -1;
}

// Lanes of the wave that are valid and hold the same key as this lane (bits of key
// above nbits must be zero).
__device__ __forceinline__ unsigned long long same_key_lanes(int key, bool valid, int nbits) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ void __launch_bounds__(kCapThreads)
route_capacity_kernel(const int32_t* __restrict__ ids, const float* __restrict__ gates, int T, int E, int k,
                      int32_t base, int adaptive, int32_t* __restrict__ limits, int32_t* __restrict__ assign,
                      float* __restrict__ weight, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token) {
  __shared__ int32_t s_cnt[kCapMaxE];
  __shared__ int32_t s_lim[kCapMaxE];
  __shared__ int32_t s_ids2[2][kCapStageSlots];  // two staging buffers: waves 1-3 fill one
  __shared__ float s_g2[2][kCapStageSlots];       // while wave 0 decides from the other
  const int tid = threadIdx.x, lane = tid & 63;
  const bool decider = tid < 64;

  for (int e = tid; e < E; e += kCapThreads) {
    s_cnt[e] = 0;
    s_lim[e] = limits[e];
  }
  const int per_pass = kCapStageSlots / k;  // k <= 32: at least 128 tokens
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int npass = (T + per_pass - 1) / per_pass;
  auto stage = [&](int p, int buf, int first, int nthr) {
    const int tb = p * per_pass, nt = min(per_pass, T - tb);
    const long long s0 = (long long)tb * k;
    for (int s = tid - first; s < nt * k; s += nthr) {
      s_ids2[buf][s] = ids[s0 + s];
      s_g2[buf][s] = gates[s0 + s];
    }
  };
  if (npass > 0) stage(0, 0, 0, kCapThreads);
  for (int p = 0; p < npass; ++p) {
    __syncthreads();  // pass p is staged; the buffer staged next was last read in pass p - 1
    const int buf = p & 1;
    if (!decider) {
      if (p + 1 < npass) stage(p + 1, buf ^ 1, 64, kCapThreads - 64);
      continue;
    }
    const int tb = p * per_pass, nt = min(per_pass, T - tb);
    const int32_t* s_ids = s_ids2[buf];
    const float* s_g = s_g2[buf];
    int t = 0;
    while (t < nt) {
      const int i = t + lane;
      const bool act = i < nt;
      int slot = 0, cnt = 0, lim = 0;
      const int e_sel = act ? first_with_room(s_ids, s_cnt, s_lim, i, k, E, &slot, &cnt, &lim) : -2;
      const unsigned long long same = same_key_lanes(e_sel, e_sel >= 0, nbits);
      const int rank = __popcll(same & lanes_below(lane));
      const bool bad = act && (e_sel < 0 || cnt + rank >= lim);
      const unsigned long long badm = __ballot(bad);
      const int stop = badm ? __ffsll(badm) - 1 : 64;
      if (act && lane < stop) {
        assign[tb + i] = e_sel | (cnt + rank) << kPosShift;
        weight[tb + i] = s_g[i * k + slot];
        atomicAdd(&s_cnt[e_sel], 1);
      }
      if (stop == 64) {
        t += 64;
        continue;
      }
      if (stop > 0 && __shfl(e_sel, stop) >= 0) {  // its expert filled inside the chunk: start there
        t += stop;
        continue;
      }
      // every preference of token t + stop is full (counts only grow): least-loaded rule
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      const int is = t + stop;
      int bc = INT_MAX, bi = INT_MAX;
      for (int e = lane; e < E; e += 64) {
        const int c = s_cnt[e];
        if (c < bc) {
          bc = c;
          bi = e;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const int oc = __shfl_xor(bc, off), oi = __shfl_xor(bi, off);
        if (oc < bc || (oc == bc && oi < bi)) {
          bc = oc;
          bi = oi;
        }
      }
      const bool take = 2ll * bc < 3ll * s_lim[bi];
      if (lane == 0) {
        assign[tb + is] = take ? bi | bc << kPosShift : -1;
        weight[tb + is] = take ? 0.5f * s_g[is * k] : 0.0f;
        if (take) s_cnt[bi] = bc + 1;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      t = is + 1;
    }
  }
  __syncthreads();

  if (adaptive)
    for (int e = tid; e < E; e += kCapThreads) {
      const long long c = s_cnt[e], L = s_lim[e];
      long long n = L;
      if (c >= L)
        n = min(6 * L / 5, (long long)INT_MAX);
      else if (2 * c < L)
        n = max((long long)base, 9 * L / 10);
      limits[e] = (int32_t)n;
    }
  __syncthreads();  // s_lim becomes the offsets below
  if (decider) {
    // exclusive scan of the counts: each lane sums a run of experts, then a wave scan
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int sum = 0;
    for (int u = 0; u < per; ++u)
      if (e0 + u < E) sum += s_cnt[e0 + u];
    int inc = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(inc, off);
      if (lane >= off) inc += v;
    }
    int run = inc - sum;
    for (int u = 0; u < per; ++u)
      if (e0 + u < E) {
        offsets[e0 + u] = run;
        s_lim[e0 + u] = run;
        run += s_cnt[e0 + u];
      }
    if (lane == 63) offsets[E] = inc;
  }
  __syncthreads();

  // place each kept token at its expert's offset plus its place, and unpack assign
  for (int t = tid; t < T; t += kCapThreads) {
    const int v = assign[t];
    if (v < 0) continue;
    const int e = v & ((1 << kPosShift) - 1);
    const int pos = (e < E ? s_lim[e] : T) + (v >> kPosShift);
    if ((unsigned)pos < (unsigned)T) sorted_token[pos] = t;
    assign[t] = e;
  }
}

// Route of a capacity result for the expert FFN: slot 0 of each token carries its
// expert and weight, the other slots gate 0 (the combine skips them); a dropped token
// has gate 0 everywhere.  Unused pair positions point at row 0, which always exists.
__global__ void route_from_capacity_slots_kernel(const int32_t* __restrict__ assign, const float* __restrict__ weight,
                                                 const int32_t* __restrict__ cap_offsets, int T, int E, int k,
                                                 int32_t* __restrict__ ids, float* __restrict__ gates,
                                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ pair_pos) {
  const long long p = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p <= E) {
    offsets[p] = cap_offsets[p];
    if (p < E) counts[p] = cap_offsets[p + 1] - cap_offsets[p];
  }
  if (p >= (long long)T * k) return;
  const int t = (int)(p / k), j = (int)(p - (long long)t * k);
  ids[p] = j == 0 ? assign[t] : -1;
  gates[p] = j == 0 ? weight[t] : 0.0f;
  pair_pos[p] = 0;
}

__global__ void route_from_capacity_rows_kernel(const int32_t* __restrict__ cap_offsets,
                                                const int32_t* __restrict__ sorted_token, int T, int E, int k,
                                                int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= T || r >= cap_offsets[E]) return;
  const int t = sorted_token[r];
  if ((unsigned)t >= (unsigned)T) return;
  sorted_pair[r] = t * k;
  pair_pos[(size_t)t * k] = r;
}

}  // namespace

hipError_t launch_route_from_capacity(const int32_t* assign, const float* weight, const int32_t* cap_offsets,
                                      const int32_t* sorted_token, int T, int E, int k, int32_t* ids, float* gates,
                                      int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                      hipStream_t st) {
  if (E < 1 || k < 1 || T < 0 || (long long)T * k >= (1ll << 31)) return hipErrorInvalidValue;
  const long long slots = (long long)T * k > E + 1 ? (long long)T * k : E + 1;
  route_from_capacity_slots_kernel<<<(unsigned)((slots + 255) / 256), 256, 0, st>>>(
      assign, weight, cap_offsets, T, E, k, ids, gates, counts, offsets, pair_pos);
  if (T > 0)
    route_from_capacity_rows_kernel<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(cap_offsets, sorted_token, T, E,
                                                                                  k, sorted_pair, pair_pos);
  return hipGetLastError();
}

hipError_t launch_route_capacity(const int32_t* ids, const float* gates, int T, int E, int k, int32_t base,
                                 int adaptive, int32_t* limits, int32_t* assign, float* weight, int32_t* offsets,
                                 int32_t* sorted_token, hipStream_t st) {
  if (E < 1 || E > kCapMaxE || k < 1 || k > 32 || T < 0 || T > kCapMaxTokens) return hipErrorInvalidValue;
  route_capacity_kernel<<<1, kCapThreads, 0, st>>>(ids, gates, T, E, k, base, adaptive, limits, assign, weight,
                                                   offsets, sorted_token);
  return hipGetLastError();
}

}  // namespace afd
