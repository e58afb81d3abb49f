// Grouped expert GEMMs in bf16 on the gfx950 matrix cores, weight-streaming form.
//
// The expert FFN's dominant cost is reading expert weights that only a few tokens
// use ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §1: each expert's weight
// matrices are large but a step activates them with few tokens; MoE FFN utilisation
// falls from 28% at batch 395 to 0.5% at batch 6).  This kernel is built for that
// regime: one wave computes a 16-row tile (the tokens of one expert, padded) times
// 32 output columns over the whole reduction, streaming that column group's
// pre-packed weight fragments straight from HBM into registers: every lane issues
// 16-byte loads that together cover contiguous 1 KiB fragments, two fragments per
// 32-deep step, loaded eight steps ahead of use (nontemporal), and each fragment feeds one
// v_mfma_f32_16x16x32_bf16 directly (no LDS round trip: each weight byte is used by
// exactly one wave).  The 16 activation rows of the tile are gathered through the
// expert-sorted pair order (tokens of x for the gate/up projection, intermediate
// rows for the down projection).
//
//   gate/up (SWIGLU = true): the column group holds gate block j and up block j, so
//     the epilogue forms h = SiLU(gate) * up in registers and stores bf16 h;
//   down    (SWIGLU = false): the group holds output blocks 2j and 2j+1, stored as
//     bf16 rows for the combine (which sums them in fp32).
// MFMA operand order (16x16x32 bf16): lane l supplies row (l % 16) of A and column
// (l % 16) of B at reduction offsets (l / 16) * 8 .. + 7; it receives rows
// (l / 16) * 4 .. + 3 of column (l % 16) of the 16x16 fp32 result.
#include "grouped.h"

namespace afd {

constexpr int kGemmThreads = 256;
constexpr int kGemmWaves = kGemmThreads / kWave;

// Weight fragments are read exactly once per launch: load them nontemporally so they
// stream past the caches instead of evicting the activation rows every wave re-reads.
__device__ __forceinline__ bf16x8 load_weight_frag(const i32x4* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(p));
}

// acc0/acc1 += A[16 x K] * B[K x 32] over K = 32 * KB, with the loads of step s + D
// issued while step s computes (a rotating register pipeline; no branch inside, so
// the compiler waits only for the oldest outstanding loads).  KB % D == 0, KB >= D.
template <int D>
__device__ __forceinline__ void stream_mfma(const bf16x8* __restrict__ A, const i32x4* __restrict__ B, int KB,
                                            f32x4& acc0, f32x4& acc1) {
  bf16x8 a[D], b0[D], b1[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    a[u] = A[u * 4];
    b0[u] = load_weight_frag(B + (u * 2) * 64);
    b1[u] = load_weight_frag(B + (u * 2 + 1) * 64);
  }
  for (int s0 = D; s0 < KB; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
      const int s = s0 + u;
      a[u] = A[s * 4];
      b0[u] = load_weight_frag(B + (s * 2) * 64);
      b1[u] = load_weight_frag(B + (s * 2 + 1) * 64);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
  }
}

// Weights of the first D steps of an item's column group, loaded ahead of its
// activations (the fused decode launch issues them before its grid barrier).
template <int D>
__device__ __forceinline__ void prime_weights(const i32x4* __restrict__ B, bf16x8* b0, bf16x8* b1) {
#pragma unroll
  for (int u = 0; u < D; ++u) {
    b0[u] = load_weight_frag(B + (u * 2) * 64);
    b1[u] = load_weight_frag(B + (u * 2 + 1) * 64);
  }
}

// stream_mfma with the weights of the first D steps already in b0 / b1.
template <int D>
__device__ __forceinline__ void stream_mfma_primed(const bf16x8* __restrict__ A, const i32x4* __restrict__ B,
                                                   int KB, f32x4& acc0, f32x4& acc1, bf16x8* b0, bf16x8* b1) {
  bf16x8 a[D];
#pragma unroll
  for (int u = 0; u < D; ++u) a[u] = A[u * 4];
  for (int s0 = D; s0 < KB; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
      const int s = s0 + u;
      a[u] = A[s * 4];
      b0[u] = load_weight_frag(B + (s * 2) * 64);
      b1[u] = load_weight_frag(B + (s * 2 + 1) * 64);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b0[u], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b1[u], acc1, 0, 0, 0);
  }
}

// Operand addresses of one work item for this lane: A row of the tile (rows past the
// tile end repeat its first row; their results are not stored) and the column group's
// weight stream.
struct StreamOps {
  const bf16x8* A;
  const i32x4* B;
  int KB;
};
// The lane's A operand stream when its tile row is activation row `arow`.
__device__ __forceinline__ const bf16x8* stream_a(const GroupedGemm& g, const Item& it, int lane, int arow) {
  const int lda = it.shared ? g.lda_shared : g.lda_routed;
  return reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(it.shared ? g.a_shared : g.a_routed) +
                                         (size_t)arow * lda) +
         (lane >> 4);
}
// Operands with A read from row `row` of the segment's rows (tiles that are not
// gathered), and the weights.
__device__ __forceinline__ StreamOps stream_ops_rows(const GroupedGemm& g, const Item& it, int lane, int row) {
  const int K = it.shared ? g.K_shared : g.K_routed;
  StreamOps o;
  o.A = stream_a(g, it, lane, row);
  const __bf16* wbase = it.shared ? static_cast<const __bf16*>(g.w_shared)
                                  : static_cast<const __bf16*>(g.w_routed) + (size_t)it.seg * g.w_expert_elems;
  o.KB = K / 32;
  o.B = reinterpret_cast<const i32x4*>(wbase) + (size_t)it.group * o.KB * 128 + lane;
  return o;
}

__device__ __forceinline__ StreamOps stream_ops(const GroupedGemm& g, const Item& it, int lane) {
  const int r = lane & 15;
  const int row = it.row0 + (r < it.nrows ? r : 0);
  StreamOps o = stream_ops_rows(g, it, lane, row);
  if (!it.shared && g.gather_routed) o.A = stream_a(g, it, lane, g.sorted_pair[row] / g.k);
  return o;
}

// Epilogue of one item: SwiGLU h rows (gate/up) or expert output rows O (down), bf16.
// gates != NULL (down only): routed rows are stored already multiplied by their pair's
// gate, so the combine sums them unweighted.
template <bool SWIGLU>
__device__ __forceinline__ void stream_store(const GroupedGemm& g, const Item& it, int lane, const f32x4& acc0,
                                             const f32x4& acc1, const float* gates) {
  const int col = lane & 15;
  const int rbase = (lane >> 4) * 4;
  __bf16* out = static_cast<__bf16*>(it.shared ? g.out_shared : g.out_routed);
  const int ldo = it.shared ? g.ldo_shared : g.ldo_routed;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + i;
    if (row >= it.nrows) continue;
    if (SWIGLU) {
      out[(size_t)(it.row0 + row) * ldo + it.group * 16 + col] = f32_to_bf16(silu(acc0[i]) * acc1[i]);
    } else {
      const float gs = gates && !it.shared ? gates[g.sorted_pair[it.row0 + row]] : 1.f;
      __bf16* o = out + (size_t)(it.row0 + row) * ldo + it.group * 32 + col;
      o[0] = f32_to_bf16(gs * acc0[i]);
      o[16] = f32_to_bf16(gs * acc1[i]);
    }
  }
}

template <bool SWIGLU>
__global__ void __launch_bounds__(kGemmThreads) gemm_bf16_stream_kernel(GroupedGemm g) {
  __shared__ SegTable tab;
  __shared__ int scan_tmp[kGemmWaves + 1];
  const int total = build_item_prefix(g, kTileRows, tab, scan_tmp);
  const int lane = lane_id();
  const int waves_in_launch = gridDim.x * kGemmWaves;
  const int wave = blockIdx.x * kGemmWaves + threadIdx.x / kWave;

  for (int item = wave; item < total; item += waves_in_launch) {
    const Item it = decode_item(g, kTileRows, tab, item);
    // The weight stream starts before the lane's activation row is known: its
    // sorted_pair entry is loaded first (an in-bounds entry is read for every tile, used
    // only when the tile's rows are gathered), then the first weight steps, so that the
    // wait for the entry does not include the weights.
    const int r = lane & 15;
    const int row = it.row0 + (r < it.nrows ? r : 0);
    const int pair = g.sorted_pair[row];
    const StreamOps o = stream_ops_rows(g, it, lane, row);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 b0[8], b1[8];
    const bool gather = !it.shared && g.gather_routed;
    if (o.KB % 8 == 0) {
      prime_weights<8>(o.B, b0, b1);
      __builtin_amdgcn_sched_barrier(0);  // the weight loads issue before the use of `pair`
      stream_mfma_primed<8>(gather ? stream_a(g, it, lane, pair / g.k) : o.A, o.B, o.KB, acc0, acc1, b0, b1);
    } else {
      prime_weights<4>(o.B, b0, b1);
      __builtin_amdgcn_sched_barrier(0);  // the weight loads issue before the use of `pair`
      stream_mfma_primed<4>(gather ? stream_a(g, it, lane, pair / g.k) : o.A, o.B, o.KB, acc0, acc1, b0, b1);
    }
    stream_store<SWIGLU>(g, it, lane, acc0, acc1, nullptr);
  }
}

// The decode layer's two grouped GEMMs in one persistent launch (the single-launch
// expert kernel of "大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §5, MegaMoE, and
// the persistent, tile-scheduled expert kernel of the ExpertPlex summary in
// "AF分离论文串讲"): every wave runs its gate/up items, loads the weights of its first
// down item's first steps (they do not depend on h), and passes a grid-wide barrier
// once every workgroup has stored its h rows; then the down items run, with each
// routed row's gate applied in the epilogue.
//
// The barrier: after a workgroup barrier, one thread makes the workgroup's h stores
// visible device-wide (agent-scope release fence), counts the workgroup in `sync[0]`
// and polls (sleeping between polls) until all gridDim.x workgroups have arrived, then
// takes an agent-scope acquire fence.  Measured on MI355X at the starved-decode layer
// (T=6): the launch takes 296 us against 212 us for the two separate GEMM launches
// (with two fences per workgroup 321 us; with h written through and no fences 268 us;
// polling 32x less often ~8 us less), so the separate launches stay the default.
// The spin is bounded: after `spin_limit` polls (~0.1-1 s at the default) it gives up,
// sets status[0] = 1 and the workgroup writes NaN into the rows of its down items
// instead of computing them, so every token those rows feed gets a NaN output (a loud
// failure, not a silently wrong one), and every wave exits.  The grid is the device's resident workgroup count (occupancy
// query at handle creation), so the workgroups are co-resident when nothing else runs
// on the device.  The counters are returned to zero by the last workgroup to leave
// (sync[1] counts departures), so consecutive launches, and replays of a captured
// launch, start from zero without a memset.  Two launches that overlap on one set of
// counters (one handle's workspace) race.  Needs K % 256 == 0 for every segment (both
// phases use 8-step rings; checked by the host).
__global__ void __launch_bounds__(kGemmThreads) gemm_bf16_fused_kernel(GroupedGemm g1, GroupedGemm g2,
                                                                       const float* gates, unsigned* sync,
                                                                       int* status, unsigned spin_limit) {
  __shared__ SegTable prefix1;
  __shared__ SegTable prefix2;
  __shared__ int scan_tmp[kGemmWaves + 1];
  __shared__ int passed;
  const int total1 = build_item_prefix(g1, kTileRows, prefix1, scan_tmp);
  const int total2 = build_item_prefix(g2, kTileRows, prefix2, scan_tmp);
  const int lane = lane_id();
  const int waves_in_launch = gridDim.x * kGemmWaves;
  const int wave = blockIdx.x * kGemmWaves + threadIdx.x / kWave;

  for (int item = wave; item < total1; item += waves_in_launch) {
    const Item it = decode_item(g1, kTileRows, prefix1, item);
    const StreamOps o = stream_ops(g1, it, lane);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    stream_mfma<8>(o.A, o.B, o.KB, acc0, acc1);
    stream_store<true>(g1, it, lane, acc0, acc1, nullptr);
  }

  // the first down item's weights, ahead of the barrier
  bf16x8 b0[8], b1[8];
  Item first = {};
  const bool has_first = wave < total2;
  if (has_first) {
    first = decode_item(g2, kTileRows, prefix2, wave);
    prime_weights<8>(stream_ops(g2, first, lane).B, b0, b1);
  }

  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    atomicAdd(&sync[0], 1u);
    unsigned polls = 0;
    int ok = 1;
    while (__hip_atomic_load(&sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x) {
      __builtin_amdgcn_s_sleep(64);
      if (++polls > spin_limit) {
        ok = 0;
        atomicExch(status, 1);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    passed = ok;
  }
  __syncthreads();

  if (passed) {
    if (has_first) {
      const StreamOps o = stream_ops(g2, first, lane);
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      stream_mfma_primed<8>(o.A, o.B, o.KB, acc0, acc1, b0, b1);
      stream_store<false>(g2, first, lane, acc0, acc1, gates);
    }
    for (int item = wave + waves_in_launch; item < total2; item += waves_in_launch) {
      const Item it = decode_item(g2, kTileRows, prefix2, item);
      const StreamOps o = stream_ops(g2, it, lane);
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      stream_mfma<8>(o.A, o.B, o.KB, acc0, acc1);
      stream_store<false>(g2, it, lane, acc0, acc1, gates);
    }
  } else {
    const float nan = __builtin_nanf("");
    const f32x4 q = {nan, nan, nan, nan};
    for (int item = wave; item < total2; item += waves_in_launch)
      stream_store<false>(g2, decode_item(g2, kTileRows, prefix2, item), lane, q, q, gates);
  }

  // the last workgroup to leave returns both counters to zero
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned d = atomicAdd(&sync[1], 1u);
    if (d == gridDim.x - 1) {
      atomicExch(&sync[0], 0u);
      atomicExch(&sync[1], 0u);
    }
  }
}

hipError_t launch_gemm_bf16_fused(const GroupedGemm& g1, const GroupedGemm& g2, const float* gates, unsigned* sync,
                                  int* status, int resident_blocks, unsigned spin_limit, hipStream_t st) {
  if (g1.K_routed % 256 || g2.K_routed % 256 || (g1.shared_rows > 0 && (g1.K_shared % 256 || g2.K_shared % 256)))
    return hipErrorInvalidValue;
  if (resident_blocks <= 0) return hipErrorInvalidValue;
  gemm_bf16_fused_kernel<<<(unsigned)resident_blocks, kGemmThreads, 0, st>>>(g1, g2, gates, sync, status,
                                                                             spin_limit);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st) {
  if (max_items <= 0) return hipSuccess;
  // persistent grid of resident workgroups only: a workgroup that waits for a free
  // slot would start its items a whole item late
  long long blocks = (max_items + kGemmWaves - 1) / kGemmWaves;
  if (blocks > max_blocks) blocks = max_blocks;
  if (swiglu)
    gemm_bf16_stream_kernel<true><<<(unsigned)blocks, kGemmThreads, 0, st>>>(g);
  else
    gemm_bf16_stream_kernel<false><<<(unsigned)blocks, kGemmThreads, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace afd

namespace afd {
hipError_t gemm_occupancy_bf16(int* gate_up, int* down) {
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(gate_up, gemm_bf16_stream_kernel<true>, kGemmThreads, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(down, gemm_bf16_stream_kernel<false>, kGemmThreads, 0);
  return e;
}
hipError_t gemm_occupancy_bf16_fused(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, gemm_bf16_fused_kernel, kGemmThreads, 0);
}
}  // namespace afd
