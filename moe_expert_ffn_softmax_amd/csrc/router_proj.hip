// Router projection: the scores the top-k router selects on, computed from the
// hidden states.  The router of "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态
// 专家放置" (§4.1) is a bias-free linear map from the hidden size to the experts plus a
// per-expert dynamic bias, added before the top-k:
//   logits[t, e] = sum_h x[t, h] * W[e, h] + bias[e]   (fp32 accumulation),
// W stored [E, H] (row e: expert e's gate vector).
//
// bf16 (the bf16 and fp8 layers), on v_mfma_f32_16x16x32_bf16: lane l supplies token
// (l % 16) of A and expert (l % 16) of B at reduction offsets (l / 16) * 8 .. + 7, i.e.
// 16 contiguous bytes of an x row and of a W row, so both operands come from their
// natural row-major layouts; the lane receives tokens (l / 16) * 4 .. + 3 of expert
// (l % 16).
//   * Up to 64 tokens (decode): one workgroup per 16-token x 16-expert tile, its four
//     waves splitting the reduction (wave w takes the 32-deep steps s = w mod 4) with
//     loads several steps ahead; the four partial tiles meet in LDS and are summed in
//     wave order.  E / 16 workgroups per token tile stream W in parallel.
//   * More tokens: one workgroup per 64-token x 64-expert tile.  The tile's W rows
//     are staged through LDS 128 deep at a time (double-buffered, one barrier per
//     stage) and shared by the four waves, each of which owns 16 tokens and loads its
//     x fragments straight into registers; both streams run four stages ahead in
//     register rings.
// fp32 (the fp32 layer): one thread per (token, expert), a sequential fp32 FMA chain.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kProjWaves = 4;
constexpr int kProjThreads = kProjWaves * kWave;
constexpr int kProjSmallTokens = 64;  // token counts up to this use the split-reduction kernel
constexpr int kProjAhead = 6;         // steps in flight per wave in the split-reduction kernel

__global__ void __launch_bounds__(kProjThreads) router_proj_small_kernel(const __bf16* __restrict__ x,
                                                                         const __bf16* __restrict__ w,
                                                                         const float* __restrict__ bias, int T, int H,
                                                                         int E, float* __restrict__ logits) {
  __shared__ f32x4 part[kProjWaves][kWave];
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int ntt = (T + 15) / 16;
  const int tt = blockIdx.x % ntt, et = blockIdx.x / ntt;
  const int t = tt * 16 + (lane & 15), e = et * 16 + (lane & 15);
  const int tc = t < T ? t : T - 1, ec = e < E ? e : E - 1;
  const bf16x8* A = reinterpret_cast<const bf16x8*>(x + (size_t)tc * H) + (lane >> 4);
  const bf16x8* B = reinterpret_cast<const bf16x8*>(w + (size_t)ec * H) + (lane >> 4);
  const int n = H / 128;  // this wave's steps: s = wv + 4 i, i < n (H / 32 steps in all)

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bf16x8 a[kProjAhead], b[kProjAhead];
#pragma unroll
  for (int u = 0; u < kProjAhead; ++u) {
    const int i = u < n ? u : n - 1;
    a[u] = A[(wv + 4 * i) * 4];
    b[u] = B[(wv + 4 * i) * 4];
  }
  // ring slot u holds step i0 + u; past the end the loads repeat the last step and
  // their products are not accumulated
  for (int i0 = 0; i0 < n; i0 += kProjAhead) {
#pragma unroll
    for (int u = 0; u < kProjAhead; ++u) {
      if (i0 + u < n) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
      int i = i0 + u + kProjAhead;
      i = i < n ? i : n - 1;
      a[u] = A[(wv + 4 * i) * 4];
      b[u] = B[(wv + 4 * i) * 4];
    }
  }
  part[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && e < E) {
    f32x4 s = part[0][lane];
#pragma unroll
    for (int v = 1; v < kProjWaves; ++v) {
      const f32x4 p = part[v][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += p[i];
    }
    const float bv = bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tt * 16 + (lane >> 4) * 4 + i;
      if (tok < T) logits[(size_t)tok * E + e] = s[i] + bv;
    }
  }
}

constexpr int kPT = 64;                      // tokens per workgroup (16 per wave)
constexpr int kPE = 64;                      // experts per workgroup (4 blocks of 16)
constexpr int kPSteps = 4;                   // 32-deep steps per stage (128 deep)
constexpr int kPStage = kPSteps * kPE * 64;  // bytes of W per stage (16 KiB)
constexpr int kPLoads = kPStage / 16 / kProjThreads;  // 16-byte W loads per thread and stage (4)
constexpr int kPAhead = 4;                   // stages of W and x in flight (even: LDS buffer = stage % 2)

__global__ void __launch_bounds__(kProjThreads) router_proj_tiled_kernel(const __bf16* __restrict__ x,
                                                                         const __bf16* __restrict__ w,
                                                                         const float* __restrict__ bias, int T, int H,
                                                                         int E, float* __restrict__ logits) {
  // W stage layout: [step][expert block][lane][16 B], i.e. the B fragments in operand
  // order; load j of thread t fills 16-byte slot t + 256 j
  __shared__ __attribute__((aligned(16))) unsigned char ws[2][kPStage];
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int ntt = (T + kPT - 1) / kPT;
  const int tt = blockIdx.x % ntt, et = blockIdx.x / ntt;
  const int t = tt * kPT + wv * 16 + (lane & 15);
  const int tc = t < T ? t : T - 1;
  const bf16x8* A = reinterpret_cast<const bf16x8*>(x + (size_t)tc * H) + (lane >> 4);
  // this thread's W loads: slot q = threadIdx.x + 256 j -> step q / 256, expert block
  // (q / 64) % 4, lane position q % 64
  const bf16x8* Bl[kPLoads];
  int boff[kPLoads];
#pragma unroll
  for (int j = 0; j < kPLoads; ++j) {
    const int q = threadIdx.x + kProjThreads * j;
    const int l = q % 64;
    int e = et * kPE + ((q / 64) % 4) * 16 + (l % 16);
    e = e < E ? e : E - 1;
    Bl[j] = reinterpret_cast<const bf16x8*>(w + (size_t)e * H) + (l / 16);
    boff[j] = (q / 256) * 4;  // bf16x8 offset of the step inside the stage
  }
  const int NS = H / 128;

  f32x4 acc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // register rings kPAhead stages deep: wr[r] and ar[r] hold stages of residue r;
  // loads past the last stage repeat it (never used)
  bf16x8 wr[kPAhead][kPLoads], ar[kPAhead][kPSteps];
  auto load_w = [&](int s, bf16x8* dst) {
    s = s < NS ? s : NS - 1;
#pragma unroll
    for (int j = 0; j < kPLoads; ++j) dst[j] = Bl[j][s * 16 + boff[j]];
  };
  auto store_w = [&](int buf, const bf16x8* src) {
#pragma unroll
    for (int j = 0; j < kPLoads; ++j)
      *reinterpret_cast<bf16x8*>(&ws[buf][(threadIdx.x + kProjThreads * j) * 16]) = src[j];
  };
  auto load_a = [&](int s, bf16x8* dst) {
    s = s < NS ? s : NS - 1;
#pragma unroll
    for (int u = 0; u < kPSteps; ++u) dst[u] = A[s * 16 + u * 4];
  };
#pragma unroll
  for (int r = 0; r < kPAhead; ++r) {
    load_w(r, wr[r]);
    load_a(r, ar[r]);
  }
  store_w(0, wr[0]);
  load_w(kPAhead, wr[0]);
  __syncthreads();
  // stage s: W from LDS buffer s % 2, x from ar[s % kPAhead]; then stage s + 1's W
  // goes to the other buffer and both rings are refilled kPAhead stages ahead
  for (int s0 = 0; s0 < NS; s0 += kPAhead) {
#pragma unroll
    for (int r = 0; r < kPAhead; ++r) {
      const int s = s0 + r;
      const int buf = r & 1;
      if (s < NS) {
#pragma unroll
        for (int u = 0; u < kPSteps; ++u)
#pragma unroll
          for (int eb = 0; eb < 4; ++eb) {
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(&ws[buf][((u * 4 + eb) * 64 + lane) * 16]);
            acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[r][u], b, acc[eb], 0, 0, 0);
          }
      }
      load_a(s + kPAhead, ar[r]);
      store_w(buf ^ 1, wr[(r + 1) % kPAhead]);
      load_w(s + 1 + kPAhead, wr[(r + 1) % kPAhead]);
      __syncthreads();
    }
  }

#pragma unroll
  for (int eb = 0; eb < 4; ++eb) {
    const int e = et * kPE + eb * 16 + (lane & 15);
    if (e >= E) continue;
    const float bv = bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tt * kPT + wv * 16 + (lane >> 4) * 4 + i;
      if (tok < T) logits[(size_t)tok * E + e] = acc[eb][i] + bv;
    }
  }
}

__global__ void __launch_bounds__(kWave) router_proj_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ bias, int H, int E,
                                                                float* __restrict__ logits) {
  const int t = blockIdx.x;
  const int e = blockIdx.y * kWave + threadIdx.x;
  if (e >= E) return;
  const float* xr = x + (size_t)t * H;
  const float* wr = w + (size_t)e * H;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
  logits[(size_t)t * E + e] = acc + (bias ? bias[e] : 0.f);
}

hipError_t launch_router_proj(const void* x, const void* w, const float* bias, int T, int H, int E, bool f32,
                              float* logits, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (H % 128 || E <= 0) return hipErrorInvalidValue;
  if (f32) {
    const dim3 grid((unsigned)T, (unsigned)((E + kWave - 1) / kWave));
    router_proj_f32_kernel<<<grid, kWave, 0, st>>>(static_cast<const float*>(x), static_cast<const float*>(w),
                                                   bias, H, E, logits);
    return hipGetLastError();
  }
  const __bf16* xb = static_cast<const __bf16*>(x);
  const __bf16* wb = static_cast<const __bf16*>(w);
  if (T <= kProjSmallTokens) {
    const long long blocks = (long long)((T + 15) / 16) * ((E + 15) / 16);
    router_proj_small_kernel<<<(unsigned)blocks, kProjThreads, 0, st>>>(xb, wb, bias, T, H, E, logits);
  } else {
    const long long blocks = (long long)((T + kPT - 1) / kPT) * ((E + kPE - 1) / kPE);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    router_proj_tiled_kernel<<<(unsigned)blocks, kProjThreads, 0, st>>>(xb, wb, bias, T, H, E, logits);
  }
  return hipGetLastError();
}

}  // namespace afd
