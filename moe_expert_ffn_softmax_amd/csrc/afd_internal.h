// Host-side internals of the expert-FFN library: the handle and the kernel
// launchers each kernel file provides.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "afd_ffn.h"

namespace afd {

// Rows of one matrix-core tile of the grouped GEMMs (the token dimension).
constexpr int kTileRows = 16;
// Output columns of one work item: two 16-column blocks (gate + up for the gate/up
// projection, two adjacent blocks for the down projection).
constexpr int kGroupCols = 32;

// A grouped GEMM over the routed experts plus, optionally, the shared expert.
// Segment s < E is routed expert s: rows offsets[s] .. offsets[s] + counts[s] of the
// expert-sorted order; segment E (when shared_rows > 0) is the shared expert over
// all tokens.  Row r of a routed segment reads A row a_index(r) where
// a_index = sorted_pair[r] / k when gather_routed is set (tokens) and r otherwise
// (intermediate rows already in sorted order).
struct GroupedGemm {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  int E, k;
  int gather_routed;
  int shared_rows;              // 0 = no shared segment
  int K_routed, K_shared;       // reduction length
  int groups_routed, groups_shared;  // 32-column items per row tile
  const void* w_routed;         // packed weights of expert 0
  size_t w_expert_elems;        // packed elements per expert
  const void* w_shared;
  const float* s_routed;        // fp8 block scales (packed), else null
  size_t s_expert_elems;
  const float* s_shared;
  const void* a_routed;         // A matrices
  const void* a_shared;
  const float* as_routed;       // fp8 activation scales [rows, K/128], else null
  const float* as_shared;
  int lda_routed, lda_shared;   // A row stride (elements)
  void* out_routed;             // output rows in sorted order: h (bf16 layer: bf16, fp8
                                //   layer: fp32 or e4m3 codes), or O (bf16; fp32 layer fp32)
  void* out_shared;
  float* outs_routed;           // set: the fp8 tiled gate/up GEMM writes e4m3 codes to
  float* outs_shared;           // out_* and per-row per-128 scales here, else fp32 h
  int ldo_routed, ldo_shared;   // output row stride (elements)
};

// sel_bias [E] (or NULL): a bias added to the logits for the choice of experts only.
hipError_t launch_router(const float* logits, const float* sel_bias, int T, int E, int k, int32_t* ids,
                         float* gates, hipStream_t st);
// logits [T, E] = x [T, H] * w [E, H]^T (+ bias [E]); x and w bf16, or fp32 when f32.
hipError_t launch_router_proj(const void* x, const void* w, const float* bias, int T, int H, int E, bool f32,
                              float* logits, hipStream_t st);
// Router and permute as one launch for batches of at most route_small_tokens() tokens.
hipError_t launch_route_small(const float* logits, const float* sel_bias, int T, int E, int k, int32_t* ids,
                              float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                              int32_t* pair_pos, hipStream_t st);
int route_small_tokens();
hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, hipStream_t st);

// Weight repack into matrix-core fragment order.  src [nmat][R][C] row-major with
// R = reduction dim.  gate_up = 1 pairs column block j with block j + C/32 (gate and
// up halves); gate_up = 0 pairs blocks 2j and 2j + 1.
hipError_t launch_pack_bf16(const uint16_t* src, uint16_t* dst, int nmat, int R, int C, int gate_up,
                            hipStream_t st);

// Upper bound of the work items of a grouped GEMM for P routed pairs and T tokens
// (row tiles of `tile_rows` times column items), known on the host without the counts.
inline long long grouped_items_bound(int P, int E, int groups_routed, int shared_rows, int groups_shared,
                                     int tile_rows) {
  long long tiles = (P + tile_rows - 1) / tile_rows + (P < E ? P : E);
  long long it = tiles * groups_routed;
  if (shared_rows > 0) it += (long long)((shared_rows + tile_rows - 1) / tile_rows) * groups_shared;
  return it;
}

// Persistent grids: `max_items` bounds the work items, `max_blocks` is the number of
// workgroups the device keeps resident at once (from the occupancy query at create).
hipError_t launch_gemm_bf16(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st);
// Decode layers: g1 (gate/up) and g2 (down) in one persistent launch of
// `resident_blocks` workgroups with a grid-wide barrier between them; routed down rows
// are multiplied by gates[pair].  sync: 2 counters that start (and are left) at zero;
// status[0] is set to 1 if a workgroup gave up waiting at the barrier (after
// spin_limit polls), and such a workgroup writes NaN into its down rows.
hipError_t launch_gemm_bf16_fused(const GroupedGemm& g1, const GroupedGemm& g2, const float* gates, unsigned* sync,
                                  int* status, int resident_blocks, unsigned spin_limit, hipStream_t st);
constexpr unsigned kFusedSpinLimit = 1u << 18;  // default polls before giving up
hipError_t gemm_occupancy_bf16_fused(int* blocks);
hipError_t launch_gemm_f32(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st);
// Large-tile variant (128-row tiles, 8 column groups per item) for experts with many
// rows; `max_blocks` as above.
// The 128-row GEMM kernels use more than the default dynamic LDS; these raise the
// limit for the current device (called once per handle at creation).
hipError_t configure_gemm_bf16_tiled();
hipError_t configure_gemm_fp8_tiled();
hipError_t launch_gemm_bf16_tiled(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks,
                                  hipStream_t st);
int tiled_rows();
int tiled_groups();

// fp8 (e4m3, fp32 block scales) streaming variant; weights packed by launch_pack_fp8,
// A = fp8 codes with per-row per-128 scales `as_*`, weight scales `s_*`; writes fp32.
hipError_t launch_gemm_fp8(const GroupedGemm& g, bool swiglu, long long max_items, int max_blocks, hipStream_t st);
// a_rows: rows of the routed A matrix (tokens when gathered, else expert-sorted rows);
// refused when a row offset of either A matrix does not fit in 32 bits.
hipError_t launch_gemm_fp8_tiled(const GroupedGemm& g, bool swiglu, long long a_rows, long long max_items,
                                 int max_blocks, hipStream_t st);
int fp8_tiled_rows();
int fp8_tiled_groups();
hipError_t launch_pack_fp8(const uint8_t* src, uint8_t* dst, int nmat, int R, int C, int gate_up, hipStream_t st);
// rows x cols activations (bf16 or fp32, row stride ld) -> e4m3 codes [rows, cols]
// and fp32 scales [rows, cols / 128].
// One row segment of the fp8 activation quantisation: rows x cols values at src (row
// stride ld) -> e4m3 codes q [rows, cols] and scales [rows, cols / 128].
struct QuantSeg {
  const void* src;
  int rows, cols, ld;
  uint8_t* q;
  float* scales;
};
hipError_t launch_quant_fp8(const void* src, int rows, int cols, int ld, bool src_bf16, uint8_t* q, float* scales,
                            hipStream_t st);
// Two segments of the same source type in one launch (s1.rows may be 0).
hipError_t launch_quant_fp8_segments(const QuantSeg& s0, const QuantSeg& s1, bool src_bf16, hipStream_t st);

// Resident workgroups per compute unit of the GEMM kernels.
hipError_t gemm_occupancy_bf16(int* gate_up, int* down);
hipError_t gemm_occupancy_f32(int* gate_up, int* down);
hipError_t gemm_occupancy_fp8(int* gate_up, int* down);

// y[t] = sum_j gate[t,j] * O[pair_pos[t*k+j]] (+ Os[t]); O, Os and y all bf16
// (bf16 = true) or all fp32.
// gates_applied: the rows already carry their gates (a slot whose gate is 0 is still
// skipped, but the others are summed unweighted).
hipError_t launch_combine(const void* O, const void* Os, const float* gates, const int32_t* pair_pos,
                          int T, int k, int H, void* y, bool bf16, hipStream_t st, bool gates_applied = false);

}  // namespace afd

// Intermediate buffers of one forward call (h, the expert outputs O, and for fp8
// layers the e4m3 codes and scales of x and h): the handle's own workspace, or for
// afd_ffn_forward_noalloc a carve-up of the library's static device scratch array.
struct afd_workspace {
  void* h_routed;
  void* h_shared;
  void* o_routed;
  void* o_shared;
  uint8_t* xq;
  float* xs;
  uint8_t* hq_routed;
  float* hs_routed;
  uint8_t* hq_shared;
  float* hs_shared;
  unsigned* fused_sync;  // barrier counters and status of the fused decode launch
};

struct afd_ffn {
  afd_ffn_config cfg;
  int device;
  int num_cus;
  // repacked weights (owned)
  void* w_gu;
  void* w_d;
  void* ws_gu;
  void* ws_d;
  size_t w_gu_expert_elems, w_d_expert_elems;
  // workspace (owned)
  void* h_routed;   // [P_max, M]
  void* h_shared;   // [T_max, Ms]
  void* o_routed;   // [P_max, H], bf16 (fp32 for the fp32 layer)
  void* o_shared;   // [T_max, H], likewise
  // fp8 layers only
  float* s_gu;        // [E, H/128, 2M/128] weight block scales (copy)
  float* s_d;         // [E, M/128, H/128]
  float* ss_gu;       // shared expert scales
  float* ss_d;
  uint8_t* xq;        // [T_max, H] e4m3 codes of x
  float* xs;          // [T_max, H/128]
  uint8_t* hq_routed; // [P_max, M]
  float* hs_routed;   // [P_max, M/128]
  uint8_t* hq_shared; // [T_max, Ms]
  float* hs_shared;   // [T_max, Ms/128]
  int gemm_blocks[6];  // resident workgroups of each GEMM kernel on the whole device
                       // (bf16 gate/up, down; fp32 gate/up, down; fp8 gate/up, down)
  int gemm_mode;       // afd_gemm_kernel: automatic, 16-row or 128-row tiles, or the fused decode launch
  int fused_blocks;    // resident workgroups of the fused decode kernel on the whole device
  unsigned fused_spin_limit;  // polls at its barrier before a workgroup gives up
  unsigned* fused_sync;  // its barrier counters [2] and status [1] (owned, zeroed at create)
  // Routes last filled by afd_ffn_route_from_capacity (keyed by their sorted_pair
  // buffer), with the batch size T: such a route keeps at most T of its T * top_k
  // pairs, so the automatic GEMM choice counts T rows for it.  Any other route call on
  // the same buffers removes the entry.
  static constexpr int kCapRoutes = 16;
  const void* cap_route[kCapRoutes];
  int cap_rows[kCapRoutes];
  int cap_next;
  size_t device_bytes;
  // profiling
  bool profiling;
  std::vector<hipEvent_t> ev_pool;
  std::vector<int> ev_stage;  // stage of each recorded (start, stop) pair
  size_t ev_used;
};
