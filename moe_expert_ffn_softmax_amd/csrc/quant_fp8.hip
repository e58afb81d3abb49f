// Activation quantisation to fp8 (OCP e4m3) per row and per 128 channels, for the
// fp8 layer: scale = amax / 448 (1 for an all-zero group), code = nearest e4m3 of
// v / scale, ties to even, both divisions IEEE fp32.  The weights of that layer carry
// one fp32 scale per 128x128 block; the activations (x before the gate/up projection
// and h before the down projection) get one per row per 128 channels, so every
// 128-deep block of a product has one scale on each side.  FP8/BF16 mixed precision
// is the omica.com.cn AFD article's §3.3 ("FP8BF16混合精度").
//
// One wave per (row, 64 * VPL channels), 16 bytes per lane.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

constexpr int kQuantThreads = 256;

// Each lane loads 16 bytes: 8 bf16 or 4 fp32 values (VPL), so a 128-channel group
// spans 128 / VPL lanes and a wave covers 64 * VPL channels of one row; the group
// amax is a max over those lanes.  One launch covers up to two row segments (the
// routed and the shared expert's h of the fp8 layer); a wave's rows all belong to one.
// A wave's work item wj: the row segment, row and first channel of its lane.
struct QuantWork {
  const QuantSeg* sg;
  int r, c0;
  bool ok;  // the lane's channels are inside the row (cols is a multiple of 128, so a
            // group is all in or all out)
};

template <bool BF16>
__global__ void __launch_bounds__(kQuantThreads) quant_fp8_kernel(QuantSeg s0, QuantSeg s1) {
  constexpr int VPL = BF16 ? 8 : 4;       // values per lane
  constexpr int LPG = 128 / VPL;          // lanes per 128-channel group
  constexpr int CPW = kWave * VPL;        // channels per wave
  constexpr int U = 2;                    // work items per wave per pass: their loads are in flight together
  const int lane = lane_id();
  const long long work0 = (long long)s0.rows * ((s0.cols + CPW - 1) / CPW);
  const long long work = work0 + (long long)s1.rows * ((s1.cols + CPW - 1) / CPW);
  const long long wave = (long long)blockIdx.x * (kQuantThreads / kWave) + threadIdx.x / kWave;
  const long long waves = (long long)gridDim.x * (kQuantThreads / kWave);
  auto locate = [&](long long wj) {
    QuantWork q;
    const bool first = wj < work0;  // uniform over the wave
    q.sg = first ? &s0 : &s1;
    const long long wi = first ? wj : wj - work0;
    const int chunks = q.sg->cols > 0 ? (q.sg->cols + CPW - 1) / CPW : 1;  // past the work: any row
    q.r = (int)(wi / chunks);
    q.c0 = (int)(wi % chunks) * CPW + lane * VPL;
    q.ok = wj < work && q.c0 < q.sg->cols;
    return q;
  };
  for (long long wj = wave; wj < work; wj += U * waves) {
    QuantWork q[U];
    float v[U][VPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      q[u] = locate(wj + u * waves);
#pragma unroll
      for (int i = 0; i < VPL; ++i) v[u][i] = 0.f;
      if (q[u].ok) {
        const QuantSeg& sg = *q[u].sg;
        if (BF16) {
          const uint4 raw =
              *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(sg.src) + (size_t)q[u].r * sg.ld + q[u].c0);
          const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[u][2 * i] = bf16_bits_to_f32((uint16_t)(wds[i] & 0xffffu));
            v[u][2 * i + 1] = bf16_bits_to_f32((uint16_t)(wds[i] >> 16));
          }
        } else {
          const float4 f =
              *reinterpret_cast<const float4*>(static_cast<const float*>(sg.src) + (size_t)q[u].r * sg.ld + q[u].c0);
          v[u][0] = f.x;
          v[u][1] = f.y;
          v[u][2] = f.z;
          v[u][3] = f.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const QuantSeg& sg = *q[u].sg;
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
#pragma unroll
      for (int off = LPG / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
      const float s = amax > 0.f ? amax / 448.f : 1.f;
      if (q[u].ok) {
        const int cols = sg.cols;
        uint32_t pk[VPL / 4];
#pragma unroll
        for (int i = 0; i < VPL / 4; ++i)
          pk[i] = e4m3_pack4(v[u][4 * i] / s, v[u][4 * i + 1] / s, v[u][4 * i + 2] / s, v[u][4 * i + 3] / s);
        if (BF16)
          *reinterpret_cast<uint2*>(sg.q + (size_t)q[u].r * cols + q[u].c0) = make_uint2(pk[0], pk[VPL / 4 - 1]);
        else
          *reinterpret_cast<uint32_t*>(sg.q + (size_t)q[u].r * cols + q[u].c0) = pk[0];
        if (lane % LPG == 0) sg.scales[(size_t)q[u].r * (cols / 128) + q[u].c0 / 128] = s;
      }
    }
  }
}

hipError_t launch_quant_fp8_segments(const QuantSeg& s0, const QuantSeg& s1, bool src_bf16, hipStream_t st) {
  if (s0.rows < 0 || s1.rows < 0) return hipErrorInvalidValue;
  if (s0.rows == 0 && s1.rows == 0) return hipSuccess;
  for (const QuantSeg* sg : {&s0, &s1})
    if (sg->rows > 0 && (sg->cols % 128 || sg->ld % 8)) return hipErrorInvalidValue;
  const int cpw = kWave * (src_bf16 ? 8 : 4);
  const long long work = (long long)s0.rows * ((s0.cols + cpw - 1) / cpw) + (long long)s1.rows * ((s1.cols + cpw - 1) / cpw);
  long long blocks = (work + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (src_bf16)
    quant_fp8_kernel<true><<<(unsigned)blocks, kQuantThreads, 0, st>>>(s0, s1);
  else
    quant_fp8_kernel<false><<<(unsigned)blocks, kQuantThreads, 0, st>>>(s0, s1);
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
