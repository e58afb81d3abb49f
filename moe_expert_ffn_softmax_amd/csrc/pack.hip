// Weight repack into matrix-core fragment order (load-time work of afd_ffn_create).
//
// A bf16 weight matrix W[R][C] (R = reduction dim, C = output columns) becomes a
// sequence of 32-column groups; inside a group, for each 32-row step kb, two 1 KiB
// fragments (one per 16-column block) in the operand order of the gfx950
// v_mfma_f32_16x16x32_bf16 B operand: lane l holds the 8 consecutive rows
// kb*32 + (l/16)*8 .. +7 of column (l%16) of the block.  A wave then loads a whole
// fragment with one coalesced 16-byte load per lane, and each group's data for the
// full reduction is one contiguous stream.
//
// Column blocks of a group: for the gate/up projection ([H, 2M], gate columns first)
// group j holds gate block j and up block j, so the SwiGLU epilogue finds both halves
// of its outputs in the same lane; for the down projection group j holds the
// adjacent blocks 2j and 2j+1.
#include "afd_device.h"
#include "afd_internal.h"

namespace afd {

__global__ void pack_bf16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int nmat, int R,
                                 int C, int gate_up) {
  // one thread per 8-element lane slot of a fragment
  const size_t slots_per_mat = (size_t)R * C / 8;
  const size_t total = slots_per_mat * nmat;
  const int KB = R / 32;
  for (size_t s = blockIdx.x * (size_t)blockDim.x + threadIdx.x; s < total; s += (size_t)gridDim.x * blockDim.x) {
    const size_t mat = s / slots_per_mat;
    size_t r = s % slots_per_mat;
    const int lane = (int)(r % 64);
    r /= 64;
    const int half = (int)(r % 2);
    r /= 2;
    const int kb = (int)(r % KB);
    const int j = (int)(r / KB);
    const int c = lane % 16;
    const int col = gate_up ? half * (C / 2) + j * 16 + c : j * 32 + half * 16 + c;
    const int row0 = kb * 32 + (lane / 16) * 8;
    const uint16_t* sp = src + mat * (size_t)R * C + (size_t)row0 * C + col;
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = sp[(size_t)i * C];
    uint16_t* dp = dst + s * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) dp[i] = v[i];
  }
}

hipError_t launch_pack_bf16(const uint16_t* src, uint16_t* dst, int nmat, int R, int C, int gate_up,
                            hipStream_t st) {
  if (R % 32 || C % 32) return hipErrorInvalidValue;
  pack_bf16_kernel<<<4096, 256, 0, st>>>(src, dst, nmat, R, C, gate_up);
  return hipGetLastError();
}

}  // namespace afd
