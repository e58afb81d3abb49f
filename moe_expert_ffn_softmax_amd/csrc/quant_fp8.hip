// Activation quantisation to fp8 (OCP e4m3) per row and per 128 channels, for the
// fp8 layer: scale = amax / 448 (1 for an all-zero group), code = nearest e4m3 of
// v / scale, ties to even, both divisions IEEE fp32.  The weights of that layer carry
// one fp32 scale per 128x128 block; the activations (x before the gate/up projection
// and h before the down projection) get one per row per 128 channels, so every
// 128-deep block of a product has one scale on each side.  FP8/BF16 mixed precision
// is the omica.com.cn AFD article's §3.3 ("FP8BF16混合精度").
//
// One wave per (row, run of U 64 * VPL-channel steps of the row): the grid's x covers
// rows (one per wave, strided past the grid), its y the runs, so a wave finds its work
// without a division and has its U 16-byte loads in flight together.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kQuantThreads = 256;
constexpr int kQuantRun = 4;  // 64 * VPL-channel steps per wave, their loads in flight together

// Each lane loads 16 bytes: 8 bf16 or 4 fp32 values (VPL), so a 128-channel group
// spans 128 / VPL lanes and a wave covers 64 * VPL channels of one row per step; the
// group amax is a max over those lanes.  One launch covers up to two row segments (the
// routed and the shared expert's h of the fp8 layer).
template <bool BF16>
__global__ void __launch_bounds__(kQuantThreads) quant_fp8_kernel(QuantSeg s0, QuantSeg s1) {
  constexpr int VPL = BF16 ? 8 : 4;       // values per lane
  constexpr int LPG = 128 / VPL;          // lanes per 128-channel group
  constexpr int CPW = kWave * VPL;        // channels per wave per step
  constexpr int U = kQuantRun;
  const int lane = lane_id();
  const int rows = s0.rows + s1.rows;
  const int wave = blockIdx.x * (kQuantThreads / kWave) + threadIdx.x / kWave;
  const int waves = gridDim.x * (kQuantThreads / kWave);
  const int cs = blockIdx.y * (U * CPW);  // the run's first channel
  for (int rr = wave; rr < rows; rr += waves) {
    // the row's segment, field by field (wave-uniform values in scalar registers)
    const bool first = rr < s0.rows;
    const int r = first ? rr : rr - s0.rows;
    const int cols = first ? s0.cols : s1.cols;
    const int ld = first ? s0.ld : s1.ld;
    const char* src = static_cast<const char*>(first ? s0.src : s1.src) + (size_t)r * ld * (BF16 ? 2 : 4);
    uint8_t* q = (first ? s0.q : s1.q) + (size_t)r * cols;
    float* scales = (first ? s0.scales : s1.scales) + (size_t)r * (cols / 128);
    if (cs < cols) {  // wave-uniform
      // Loads are branch-free (a lane past the row's end reads its first piece and
      // zeroes it), so that the U loads are in flight together: a load under a divergent
      // branch is waited for before the next one issues.
      float v[U][VPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c0 = cs + u * CPW + lane * VPL;
        const bool in = c0 < cols;  // cols is a multiple of 128: a group is all in or all out
        const int c = in ? c0 : 0;
        if (BF16) {
          const uint4 raw = *reinterpret_cast<const uint4*>(src + (size_t)c * 2);
          const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][2 * i] = in ? bf16_bits_to_f32((uint16_t)(wds[i] & 0xffffu)) : 0.f;
            v[u][2 * i + 1] = in ? bf16_bits_to_f32((uint16_t)(wds[i] >> 16)) : 0.f;
          }
        } else {
          const float4 f = *reinterpret_cast<const float4*>(src + (size_t)c * 4);
          v[u][0] = in ? f.x : 0.f;
          v[u][1] = in ? f.y : 0.f;
          v[u][2] = in ? f.z : 0.f;
          v[u][3] = in ? f.w : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c0 = cs + u * CPW + lane * VPL;
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
#pragma unroll
        for (int off = LPG / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
        const float sc = amax > 0.f ? amax / 448.f : 1.f;
        if (c0 < cols) {
          uint32_t pk[VPL / 4];
#pragma unroll
          for (int i = 0; i < VPL / 4; ++i)
            pk[i] = e4m3_pack4(v[u][4 * i] / sc, v[u][4 * i + 1] / sc, v[u][4 * i + 2] / sc, v[u][4 * i + 3] / sc);
          if (BF16)
            *reinterpret_cast<uint2*>(q + c0) = make_uint2(pk[0], pk[VPL / 4 - 1]);
          else
            *reinterpret_cast<uint32_t*>(q + c0) = pk[0];
          if (lane % LPG == 0) scales[c0 / 128] = sc;
        }
      }
    }
  }
}

hipError_t launch_quant_fp8_segments(const QuantSeg& s0, const QuantSeg& s1, bool src_bf16, hipStream_t st) {
  if (s0.rows < 0 || s1.rows < 0) return hipErrorInvalidValue;
  if (s0.rows == 0 && s1.rows == 0) return hipSuccess;
  if ((long long)s0.rows + s1.rows > 0x7fffffff) return hipErrorInvalidValue;
  for (const QuantSeg* sg : {&s0, &s1})
    if (sg->rows > 0 && (sg->cols % 128 || sg->ld % 8)) return hipErrorInvalidValue;
  // x: one wave per row, up to 32768 waves (rows beyond that are strided); y: runs of
  // kQuantRun steps of the longer segment's rows
  const long long rows = (long long)s0.rows + s1.rows;
  long long blocks = (rows + kQuantThreads / kWave - 1) / (kQuantThreads / kWave);
  if (blocks > 8192) blocks = 8192;
  const int cpw = kWave * (src_bf16 ? 8 : 4);
  const int cols = (s1.rows > 0 && s1.cols > s0.cols) || s0.rows == 0 ? s1.cols : s0.cols;
  const int runs = (cols + kQuantRun * cpw - 1) / (kQuantRun * cpw);
  const dim3 grid((unsigned)blocks, (unsigned)(runs > 0 ? runs : 1));
  if (src_bf16)
    quant_fp8_kernel<true><<<grid, kQuantThreads, 0, st>>>(s0, s1);
  else
    quant_fp8_kernel<false><<<grid, kQuantThreads, 0, st>>>(s0, s1);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* src, int rows, int cols, int ld, bool src_bf16, uint8_t* q, float* scales,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const QuantSeg s0 = {src, rows, cols, ld, q, scales};
  const QuantSeg none = {nullptr, 0, 128, 128, nullptr, nullptr};
  return launch_quant_fp8_segments(s0, none, src_bf16, st);
}

}  // namespace afd
