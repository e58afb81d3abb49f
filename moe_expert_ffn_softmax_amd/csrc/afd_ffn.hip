// C ABI of the expert-FFN layer: argument checks, weight repack, workspace and the
// launch sequence of route (router -> permute) and forward (gate/up GEMM + SwiGLU
// -> down GEMM -> combine), all asynchronous on the caller's stream.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "afd_internal.h"
#include "capacity.h"

namespace {

// Device scratch of afd_ffn_forward_noalloc: the intermediate buffers of one forward
// call, for callers that cannot allocate device memory.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` only names the
// symbol; kernels get its device address, looked up once per device at handle
// creation (with that device current) and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) { return fail(AFD_EHIP, "%s: %s", what, hipGetErrorString(e)); }

// Device address of `scratch` on device `dev`, which must be current.
int scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(AFD_EUNSUPPORTED, "device %d above the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return AFD_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  // the fused decode launch's barrier counters live in the first 256 bytes: zero
  e = hipMemset(p, 0, 256);
  if (e != hipSuccess) return hip_fail(e, "hipMemset(scratch counters)");
  g_scratch[dev] = p;
  return AFD_OK;
}

size_t elem_size(int dtype) { return dtype == AFD_F32 ? 4 : dtype == AFD_BF16 ? 2 : 1; }

int check_config(const afd_ffn_config* c) {
  if (!c) return fail(AFD_EINVAL, "config is NULL");
  if (c->hidden <= 0 || c->hidden % 128) return fail(AFD_EINVAL, "hidden=%d must be a positive multiple of 128", c->hidden);
  if (c->inter <= 0 || c->inter % 128) return fail(AFD_EINVAL, "inter=%d must be a positive multiple of 128", c->inter);
  if (c->shared_inter < 0 || c->shared_inter % 128)
    return fail(AFD_EINVAL, "shared_inter=%d must be 0 or a positive multiple of 128", c->shared_inter);
  if (c->num_experts < 1 || c->num_experts > 1024) return fail(AFD_EINVAL, "num_experts=%d not in [1, 1024]", c->num_experts);
  if (c->top_k < 1 || c->top_k > c->num_experts || c->top_k > 32)
    return fail(AFD_EINVAL, "top_k=%d not in [1, min(num_experts, 32)]", c->top_k);
  if (c->max_tokens < 1) return fail(AFD_EINVAL, "max_tokens=%d must be >= 1", c->max_tokens);
  if ((long long)c->max_tokens * c->top_k >= (1ll << 31)) return fail(AFD_EINVAL, "max_tokens * top_k >= 2^31");
  if (c->dtype != AFD_F32 && c->dtype != AFD_BF16 && c->dtype != AFD_FP8_E4M3)
    return fail(AFD_EINVAL, "unknown dtype %d", c->dtype);
  // the fp8 128-row GEMMs address activation rows (x: max_tokens x hidden codes; h:
  // max_tokens * top_k x inter and max_tokens x shared_inter) by 32-bit byte offsets
  if (c->dtype == AFD_FP8_E4M3) {
    const long long T = c->max_tokens;
    const long long most = std::max({T * c->hidden, T * c->top_k * c->inter, T * c->shared_inter});
    if (most >= (1ll << 32)) return fail(AFD_EINVAL, "fp8 layer: an activation matrix of max_tokens rows exceeds 4 GiB");
  }
  return AFD_OK;
}

// Is a non-null pointer off an `a`-byte boundary?  Buffers the kernels read or write
// in 16-byte vectors must be 16-byte aligned, the others 4-byte aligned.
bool misaligned(const void* p, size_t a) { return p && reinterpret_cast<uintptr_t>(p) % a != 0; }


// Do the byte ranges [a, a + na) and [b, b + nb) intersect?
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// Byte ranges of the route buffers for T tokens: ids, gates, sorted_pair, pair_pos
// [T * k], counts [E], offsets [E + 1].
struct RouteRanges {
  const void* p[6];
  size_t n[6];
};
RouteRanges route_ranges(const afd_ffn* h, const afd_route* r, int32_t T) {
  const size_t P = (size_t)T * h->cfg.top_k * 4, E = (size_t)h->cfg.num_experts * 4;
  return {{r->topk_ids, r->topk_gates, r->sorted_pair, r->pair_pos, r->expert_counts, r->expert_offsets},
          {P, P, P, P, E, E + 4}};
}

// Does [p, p + n) intersect any route buffer?
bool overlaps_route(const void* p, size_t n, const afd_ffn* h, const afd_route* r, int32_t T) {
  const RouteRanges rr = route_ranges(h, r, T);
  for (int i = 0; i < 6; ++i)
    if (overlaps(p, n, rr.p[i], rr.n[i])) return true;
  return false;
}

int check_route(const afd_ffn* h, const afd_route* r, int32_t T) {
  if (!h) return fail(AFD_EINVAL, "handle is NULL");
  if (!r) return fail(AFD_EINVAL, "route is NULL");
  if (T < 0 || T > h->cfg.max_tokens) return fail(AFD_EINVAL, "T=%d not in [0, max_tokens=%d]", T, h->cfg.max_tokens);
  if (!r->topk_ids || !r->topk_gates || !r->expert_counts || !r->expert_offsets || !r->sorted_pair || !r->pair_pos)
    return fail(AFD_EINVAL, "a route buffer is NULL");
  if (misaligned(r->topk_ids, 4) || misaligned(r->topk_gates, 4) || misaligned(r->expert_counts, 4) ||
      misaligned(r->expert_offsets, 4) || misaligned(r->sorted_pair, 4) || misaligned(r->pair_pos, 4))
    return fail(AFD_EINVAL, "route buffers must be 4-byte aligned");
  if (T > 0) {
    const RouteRanges rr = route_ranges(h, r, T);
    for (int i = 0; i < 6; ++i)
      for (int j = i + 1; j < 6; ++j)
        if (overlaps(rr.p[i], rr.n[i], rr.p[j], rr.n[j])) return fail(AFD_EINVAL, "route buffers overlap each other");
  }
  return AFD_OK;
}

void release(afd_ffn* h) {
  void* bufs[] = {h->w_gu,      h->w_d,     h->ws_gu,    h->ws_d,      h->h_routed,  h->h_shared,
                  h->o_routed,  h->o_shared, h->s_gu,    h->s_d,       h->ss_gu,     h->ss_d,
                  h->xq,        h->xs,      h->hq_routed, h->hs_routed, h->hq_shared, h->hs_shared,
                  h->fused_sync};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  for (hipEvent_t e : h->ev_pool) (void)hipEventDestroy(e);
  delete h;
}

// Brackets one kernel launch with events when profiling is on: the start event is
// recorded on construction, the stop event by done(); a scope left without done()
// (a failed launch) gives its start event back.
struct StageScope {
  afd_ffn* h;
  hipStream_t st;
  int stage;
  bool on;
  StageScope(afd_ffn* h_, hipStream_t st_, int stage_) : h(h_), st(st_), stage(stage_), on(h_->profiling) {
    while (on && h->ev_pool.size() < h->ev_used + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        on = false;
        break;
      }
      h->ev_pool.push_back(e);
    }
    if (on) (void)hipEventRecord(h->ev_pool[h->ev_used++], st);
  }
  void done() {
    if (!on) return;
    (void)hipEventRecord(h->ev_pool[h->ev_used++], st);
    h->ev_stage.push_back(stage);
    on = false;
  }
  ~StageScope() {
    if (on) --h->ev_used;
  }
};

// Kernel choice for a batch of P routed pairs, unless forced either way, from whole-layer
// times of both kernels on MI355X over batch sizes: the 16-row streaming GEMM while
// experts average at most a few routed rows, the 128-row tiled GEMM above.
//   bf16: streaming up to 8 rows per expert (E=128, H=4096: streaming 4% faster at 8
//     rows, tiled 1% faster at 9, 7% at 11, 20% at 16; E=48, H=7168 with a shared
//     expert: streaming 3% faster at 8, tiled 45% faster at 16);
//   fp8: streaming up to 12 rows per expert (E=256, H=7168: streaming 33% faster at 6
//     tokens, 10% at 12 rows; tiled 15% faster at 16; with a 2048-wide shared expert
//     streaming 2% faster at 12 rows, tiled 18% faster at 16).
bool use_tiled(const afd_ffn* h, int P) {
  if (h->gemm_mode == AFD_GEMM_STREAM || h->gemm_mode == AFD_GEMM_FUSED) return false;
  if (h->gemm_mode == AFD_GEMM_TILED) return true;
  const long long rows_per_expert = h->cfg.dtype == AFD_FP8_E4M3 ? 12 : 8;
  return (long long)P > rows_per_expert * h->cfg.num_experts;
}

// Bookkeeping of routes whose rows are fewer than T * top_k (capacity routes).
void forget_route(afd_ffn* h, const afd_route* r) {
  for (int i = 0; i < afd_ffn::kCapRoutes; ++i)
    if (h->cap_route[i] == r->sorted_pair) h->cap_route[i] = nullptr;
}
void note_capacity_route(afd_ffn* h, const afd_route* r, int T) {
  forget_route(h, r);
  h->cap_route[h->cap_next] = r->sorted_pair;
  h->cap_rows[h->cap_next] = T;
  h->cap_next = (h->cap_next + 1) % afd_ffn::kCapRoutes;
}
// Upper bound of the rows a forward on route r computes: T * top_k, or T for a route
// built from a capacity result (one expert per kept token).
int route_rows(const afd_ffn* h, const afd_route* r, int T) {
  for (int i = 0; i < afd_ffn::kCapRoutes; ++i)
    if (h->cap_route[i] == r->sorted_pair) return T < h->cap_rows[i] ? T : h->cap_rows[i];
  return T * h->cfg.top_k;
}

// fp8 layer: quantise x -> gate/up GEMM -> quantise h (in the tiled GEMM's epilogue, else a
// separate pass over fp32 h) -> down GEMM -> combine.
// x == NULL: g1 already points at caller-quantised activations (no quantisation launch).
int forward_fp8(afd_ffn* h, const afd_workspace& ws, const void* x, int T, const afd_route* r, void* y,
                hipStream_t st, const afd::GroupedGemm& g1, const afd::GroupedGemm& g2) {
  const afd_ffn_config& c = h->cfg;
  const int H = c.hidden, M = c.inter, Ms = c.shared_inter, E = c.num_experts, k = c.top_k;
  const int P = T * k;
  const int rows = route_rows(h, r, T);
  if (x) {
    StageScope s(h, st, AFD_STAGE_QUANT);
    hipError_t e = afd::launch_quant_fp8(x, T, H, H, true, ws.xq, ws.xs, st);
    if (e != hipSuccess) return hip_fail(e, "x quantisation launch");
    s.done();
  }
  const bool tiled = use_tiled(h, rows);
  long long items1, items2;
  if (tiled) {
    const int tr = afd::fp8_tiled_rows(), tg = afd::fp8_tiled_groups();
    items1 = afd::grouped_items_bound(P, E, (g1.groups_routed + tg - 1) / tg, g1.shared_rows,
                                      (g1.groups_shared + tg - 1) / tg, tr);
    items2 = afd::grouped_items_bound(P, E, (g2.groups_routed + tg - 1) / tg, g2.shared_rows,
                                      (g2.groups_shared + tg - 1) / tg, tr);
  } else {
    items1 = afd::grouped_items_bound(P, E, g1.groups_routed, g1.shared_rows, g1.groups_shared, afd::kTileRows);
    items2 = afd::grouped_items_bound(P, E, g2.groups_routed, g2.shared_rows, g2.groups_shared, afd::kTileRows);
  }
  if (tiled) {
    // the tiled gate/up GEMM quantises h in its epilogue (no fp32 h round trip)
    afd::GroupedGemm gq = g1;
    gq.out_routed = ws.hq_routed;
    gq.outs_routed = ws.hs_routed;
    gq.out_shared = ws.hq_shared;
    gq.outs_shared = ws.hs_shared;
    StageScope s(h, st, AFD_STAGE_GATE_UP);
    hipError_t e = afd::launch_gemm_fp8_tiled(gq, true, T, items1, h->num_cus, st);
    if (e != hipSuccess) return hip_fail(e, "fp8 gate/up GEMM launch");
    s.done();
  } else {
    {
      StageScope s(h, st, AFD_STAGE_GATE_UP);
      hipError_t e = afd::launch_gemm_fp8(g1, true, items1, h->gemm_blocks[4], st);
      if (e != hipSuccess) return hip_fail(e, "fp8 gate/up GEMM launch");
      s.done();
    }
    StageScope s(h, st, AFD_STAGE_QUANT);
    // routed and shared h in one launch
    const afd::QuantSeg routed = {ws.h_routed, P, M, M, ws.hq_routed, ws.hs_routed};
    const afd::QuantSeg shared = {ws.h_shared, Ms ? T : 0, Ms ? Ms : 128, Ms ? Ms : 128, ws.hq_shared, ws.hs_shared};
    hipError_t e = afd::launch_quant_fp8_segments(routed, shared, false, st);
    if (e != hipSuccess) return hip_fail(e, "h quantisation launch");
    s.done();
  }
  {
    StageScope s(h, st, AFD_STAGE_DOWN);
    hipError_t e = tiled ? afd::launch_gemm_fp8_tiled(g2, false, rows, items2, h->num_cus, st)
                         : afd::launch_gemm_fp8(g2, false, items2, h->gemm_blocks[5], st);
    if (e != hipSuccess) return hip_fail(e, "fp8 down GEMM launch");
    s.done();
  }
  {
    StageScope s(h, st, AFD_STAGE_COMBINE);
    hipError_t e = afd::launch_combine(ws.o_routed, Ms ? ws.o_shared : nullptr, r->topk_gates, r->pair_pos, T, k, H, y,
                                       true, st);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    s.done();
  }
  return AFD_OK;
}

}  // namespace

extern "C" int afd_ffn_quantize_fp8(const void* src, int32_t rows, int32_t cols, int32_t src_dtype, uint8_t* codes,
                                    float* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128) return fail(AFD_EINVAL, "rows=%d cols=%d (cols must be a multiple of 128)", rows, cols);
  if (src_dtype != AFD_F32 && src_dtype != AFD_BF16) return fail(AFD_EINVAL, "source dtype must be fp32 or bf16");
  if (rows == 0) return AFD_OK;
  if (!src || !codes || !scales) return fail(AFD_EINVAL, "a buffer is NULL");
  if (misaligned(src, 16) || misaligned(codes, 8) || misaligned(scales, 4))
    return fail(AFD_EINVAL, "src must be 16-byte aligned, codes 8-byte and scales 4-byte aligned");
  hipError_t e = afd::launch_quant_fp8(src, rows, cols, cols, src_dtype == AFD_BF16, codes, scales,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AFD_OK : hip_fail(e, "quantisation launch");
}

extern "C" const char* afd_ffn_strerror(int code) {
  switch (code) {
    case AFD_OK: return "success";
    case AFD_EINVAL: return "invalid argument";
    case AFD_EUNSUPPORTED: return "unsupported data type or shape";
    case AFD_ENOMEM: return "device memory allocation failed";
    case AFD_EHIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

extern "C" const char* afd_ffn_last_error(void) { return g_last_error; }

extern "C" int afd_ffn_create(const afd_ffn_config* cfg, const void* w_gate_up, const void* w_down,
                              const float* s_gate_up, const float* s_down, const void* ws_gate_up, const void* ws_down,
                              const float* ss_gate_up, const float* ss_down, void* stream, afd_ffn_t* out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(AFD_EINVAL, "out is NULL");
  if (!w_gate_up || !w_down) return fail(AFD_EINVAL, "expert weights are NULL");
  const bool fp8 = cfg->dtype == AFD_FP8_E4M3;
  if (!fp8 && (s_gate_up || s_down || ss_gate_up || ss_down))
    return fail(AFD_EINVAL, "block scales are only taken with fp8 weights");
  if (fp8 && (!s_gate_up || !s_down)) return fail(AFD_EINVAL, "fp8 weights need their block scales");
  if (fp8 && cfg->shared_inter > 0 && (!ss_gate_up || !ss_down))
    return fail(AFD_EINVAL, "fp8 shared expert weights need their block scales");
  if (fp8 && cfg->shared_inter == 0 && (ss_gate_up || ss_down))
    return fail(AFD_EINVAL, "shared scales given without shared_inter");
  if (cfg->shared_inter > 0 && (!ws_gate_up || !ws_down)) return fail(AFD_EINVAL, "shared expert weights are NULL");
  if (cfg->shared_inter == 0 && (ws_gate_up || ws_down)) return fail(AFD_EINVAL, "shared weights given without shared_inter");
  if (misaligned(w_gate_up, 16) || misaligned(w_down, 16) || misaligned(ws_gate_up, 16) || misaligned(ws_down, 16))
    return fail(AFD_EINVAL, "weights must be 16-byte aligned");
  if (misaligned(s_gate_up, 4) || misaligned(s_down, 4) || misaligned(ss_gate_up, 4) || misaligned(ss_down, 4))
    return fail(AFD_EINVAL, "block scales must be 4-byte aligned");
  *out = nullptr;

  afd_ffn* h = new (std::nothrow) afd_ffn();
  if (!h) return fail(AFD_ENOMEM, "host allocation of the handle failed");
  h->cfg = *cfg;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e, "hipGetDevice");
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, h->device);
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e, "hipGetDeviceProperties");
  }
  h->num_cus = prop.multiProcessorCount;
  {
    const int rc2 = scratch_address(h->device);
    if (rc2 != AFD_OK) {
      release(h);
      return rc2;
    }
  }
  e = afd::configure_gemm_bf16_tiled();
  if (e == hipSuccess) e = afd::configure_gemm_fp8_tiled();
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e, "hipFuncSetAttribute (dynamic LDS limit)");
  }
  {
    int occ[6] = {0, 0, 0, 0, 0, 0};
    e = afd::gemm_occupancy_bf16(&occ[0], &occ[1]);
    if (e == hipSuccess) e = afd::gemm_occupancy_f32(&occ[2], &occ[3]);
    if (e == hipSuccess) e = afd::gemm_occupancy_fp8(&occ[4], &occ[5]);
    if (e != hipSuccess) {
      release(h);
      return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    }
    for (int i = 0; i < 6; ++i) h->gemm_blocks[i] = (occ[i] > 0 ? occ[i] : 1) * h->num_cus;
    int fo = 0;
    e = afd::gemm_occupancy_bf16_fused(&fo);
    if (e != hipSuccess) {
      release(h);
      return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    }
    h->fused_blocks = fo * h->num_cus;
  }
  // polls at the fused decode launch's barrier before a workgroup gives up; the
  // environment can lower it to provoke the give-up path (failure-injection tests)
  h->fused_spin_limit = afd::kFusedSpinLimit;
  if (const char* v = getenv("AFD_FUSED_SPIN_LIMIT")) {
    char* end = nullptr;
    const unsigned long n = strtoul(v, &end, 10);
    if (end != v && *end == '\0' && n <= afd::kFusedSpinLimit) h->fused_spin_limit = (unsigned)n;
  }

  const size_t H = cfg->hidden, M = cfg->inter, Ms = cfg->shared_inter, E = cfg->num_experts;
  const size_t P = (size_t)cfg->max_tokens * cfg->top_k, T = cfg->max_tokens;
  const size_t es = elem_size(cfg->dtype);
  const size_t hes = cfg->dtype == AFD_BF16 ? 2 : 4;  // intermediate h: bf16, or fp32 before fp8 quantisation
  const size_t oes = cfg->dtype == AFD_F32 ? 4 : 2;    // expert outputs O: bf16 except in the fp32 layer
  h->w_gu_expert_elems = H * 2 * M;
  h->w_d_expert_elems = M * H;
  const size_t sgu_n = (H / 128) * (2 * M / 128), sd_n = (M / 128) * (H / 128);
  const size_t ssgu_n = (H / 128) * (2 * Ms / 128), ssd_n = (Ms / 128) * (H / 128);

  struct Alloc {
    void** dst;
    size_t bytes;
  } allocs[] = {
      {&h->w_gu, E * H * 2 * M * es},
      {&h->w_d, E * M * H * es},
      {&h->ws_gu, H * 2 * Ms * es},
      {&h->ws_d, Ms * H * es},
      {&h->h_routed, P * M * hes},
      {&h->h_shared, T * Ms * hes},
      {&h->o_routed, P * H * oes},
      {&h->o_shared, Ms ? T * H * oes : 0},
      {(void**)&h->s_gu, fp8 ? E * sgu_n * 4 : 0},
      {(void**)&h->s_d, fp8 ? E * sd_n * 4 : 0},
      {(void**)&h->ss_gu, fp8 ? ssgu_n * 4 : 0},
      {(void**)&h->ss_d, fp8 ? ssd_n * 4 : 0},
      {(void**)&h->xq, fp8 ? T * H : 0},
      {(void**)&h->xs, fp8 ? T * (H / 128) * 4 : 0},
      {(void**)&h->hq_routed, fp8 ? P * M : 0},
      {(void**)&h->hs_routed, fp8 ? P * (M / 128) * 4 : 0},
      {(void**)&h->hq_shared, fp8 ? T * Ms : 0},
      {(void**)&h->hs_shared, fp8 ? T * (Ms / 128) * 4 : 0},
      {(void**)&h->fused_sync, 256},
  };
  for (auto& a : allocs) {
    if (a.bytes == 0) continue;
    e = hipMalloc(a.dst, a.bytes);
    if (e != hipSuccess) {
      *a.dst = nullptr;
      release(h);
      return fail(AFD_ENOMEM, "hipMalloc of %zu bytes failed: %s", a.bytes, hipGetErrorString(e));
    }
    h->device_bytes += a.bytes;
  }

  if (cfg->dtype == AFD_BF16) {
    e = afd::launch_pack_bf16(static_cast<const uint16_t*>(w_gate_up), static_cast<uint16_t*>(h->w_gu), (int)E,
                              (int)H, (int)(2 * M), 1, st);
    if (e == hipSuccess)
      e = afd::launch_pack_bf16(static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(h->w_d), (int)E, (int)M,
                                (int)H, 0, st);
    if (e == hipSuccess && Ms)
      e = afd::launch_pack_bf16(static_cast<const uint16_t*>(ws_gate_up), static_cast<uint16_t*>(h->ws_gu), 1, (int)H,
                                (int)(2 * Ms), 1, st);
    if (e == hipSuccess && Ms)
      e = afd::launch_pack_bf16(static_cast<const uint16_t*>(ws_down), static_cast<uint16_t*>(h->ws_d), 1, (int)Ms,
                                (int)H, 0, st);
  } else if (fp8) {
    e = afd::launch_pack_fp8(static_cast<const uint8_t*>(w_gate_up), static_cast<uint8_t*>(h->w_gu), (int)E, (int)H,
                             (int)(2 * M), 1, st);
    if (e == hipSuccess)
      e = afd::launch_pack_fp8(static_cast<const uint8_t*>(w_down), static_cast<uint8_t*>(h->w_d), (int)E, (int)M,
                               (int)H, 0, st);
    if (e == hipSuccess && Ms)
      e = afd::launch_pack_fp8(static_cast<const uint8_t*>(ws_gate_up), static_cast<uint8_t*>(h->ws_gu), 1, (int)H,
                               (int)(2 * Ms), 1, st);
    if (e == hipSuccess && Ms)
      e = afd::launch_pack_fp8(static_cast<const uint8_t*>(ws_down), static_cast<uint8_t*>(h->ws_d), 1, (int)Ms,
                               (int)H, 0, st);
    if (e == hipSuccess) e = hipMemcpyAsync(h->s_gu, s_gate_up, E * sgu_n * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(h->s_d, s_down, E * sd_n * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && Ms) e = hipMemcpyAsync(h->ss_gu, ss_gate_up, ssgu_n * 4, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && Ms) e = hipMemcpyAsync(h->ss_d, ss_down, ssd_n * 4, hipMemcpyDeviceToDevice, st);
  } else {
    e = hipMemcpyAsync(h->w_gu, w_gate_up, E * H * 2 * M * es, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(h->w_d, w_down, E * M * H * es, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && Ms) e = hipMemcpyAsync(h->ws_gu, ws_gate_up, H * 2 * Ms * es, hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess && Ms) e = hipMemcpyAsync(h->ws_d, ws_down, Ms * H * es, hipMemcpyDeviceToDevice, st);
  }
  if (e == hipSuccess) e = hipMemsetAsync(h->fused_sync, 0, 256, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    release(h);
    return hip_fail(e, "weight repack");
  }
  *out = h;
  return AFD_OK;
}

extern "C" int afd_ffn_destroy(afd_ffn_t h) {
  if (h) release(h);
  return AFD_OK;
}

extern "C" size_t afd_ffn_device_bytes(afd_ffn_t h) { return h ? h->device_bytes : 0; }

extern "C" size_t afd_ffn_route_bytes(afd_ffn_t h) {
  if (!h) return 0;
  const size_t P = (size_t)h->cfg.max_tokens * h->cfg.top_k, E = h->cfg.num_experts;
  return 4 * (4 * P + 2 * E + 1);  // ids, gates, sorted_pair, pair_pos [P]; counts [E]; offsets [E + 1]
}

// Steps a1-a4 on logits already checked by the caller: router (with an optional
// selection-only bias) and the permute; one launch for decode batches.
static int route_checked(afd_ffn_t h, const float* logits, const float* sel_bias, int32_t T, const afd_route* r,
                         hipStream_t st) {
  const int E = h->cfg.num_experts, k = h->cfg.top_k;
  forget_route(h, r);
  if (T <= afd::route_small_tokens()) {
    // decode batches: router and permute in one launch (timed as the router stage)
    StageScope s(h, st, AFD_STAGE_ROUTER);
    hipError_t e = afd::launch_route_small(logits, sel_bias, T, E, k, r->topk_ids, r->topk_gates, r->expert_counts,
                                           r->expert_offsets, r->sorted_pair, r->pair_pos, st);
    if (e != hipSuccess) return hip_fail(e, "route launch");
    s.done();
    return AFD_OK;
  }
  {
    StageScope s(h, st, AFD_STAGE_ROUTER);
    hipError_t e = afd::launch_router(logits, sel_bias, T, E, k, r->topk_ids, r->topk_gates, st);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    s.done();
  }
  {
    StageScope s(h, st, AFD_STAGE_PERMUTE);
    hipError_t e = afd::launch_permute(r->topk_ids, T * k, E, r->expert_counts, r->expert_offsets, r->sorted_pair,
                                       r->pair_pos, st);
    if (e != hipSuccess) return hip_fail(e, "permute launch");
    s.done();
  }
  return AFD_OK;
}

extern "C" int afd_ffn_route(afd_ffn_t h, const float* logits, int32_t T, const afd_route* r, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!logits) return fail(AFD_EINVAL, "logits is NULL");
  if (misaligned(logits, 4)) return fail(AFD_EINVAL, "logits must be 4-byte aligned");
  if (T == 0) return AFD_OK;
  if (overlaps_route(logits, (size_t)T * h->cfg.num_experts * 4, h, r, T))
    return fail(AFD_EINVAL, "logits overlap a route buffer");
  return route_checked(h, logits, nullptr, T, r, static_cast<hipStream_t>(stream));
}

extern "C" int afd_ffn_route_select_bias(afd_ffn_t h, const float* scores, const float* bias, int32_t T,
                                         const afd_route* r, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!scores || !bias) return fail(AFD_EINVAL, "scores or bias is NULL");
  if (misaligned(scores, 4) || misaligned(bias, 4)) return fail(AFD_EINVAL, "scores and bias must be 4-byte aligned");
  if (T == 0) return AFD_OK;
  if (overlaps_route(scores, (size_t)T * h->cfg.num_experts * 4, h, r, T) ||
      overlaps_route(bias, (size_t)h->cfg.num_experts * 4, h, r, T))
    return fail(AFD_EINVAL, "scores or bias overlap a route buffer");
  return route_checked(h, scores, bias, T, r, static_cast<hipStream_t>(stream));
}

extern "C" int afd_ffn_route_capacity(afd_ffn_t h, const int32_t* ids, const float* gates, int32_t T,
                                      int32_t base_capacity, int32_t adaptive, int32_t* limits, int32_t* assign,
                                      float* weight, int32_t* offsets, int32_t* sorted_token, void* stream) {
  if (!h) return fail(AFD_EINVAL, "handle is NULL");
  const afd_ffn_config& c = h->cfg;
  if (T < 0 || T > c.max_tokens) return fail(AFD_EINVAL, "T=%d not in [0, max_tokens=%d]", T, c.max_tokens);
  if (T > afd::kCapMaxTokens) return fail(AFD_EINVAL, "T=%d above %d for capacity routing", T, afd::kCapMaxTokens);
  if (base_capacity < 0) return fail(AFD_EINVAL, "base_capacity=%d must be >= 0", base_capacity);
  if (!limits || !offsets) return fail(AFD_EINVAL, "limits or offsets is NULL");
  if (T > 0 && (!ids || !gates || !assign || !weight || !sorted_token))
    return fail(AFD_EINVAL, "ids, gates, assign, weight or sorted_token is NULL");
  const void* bufs[7] = {ids, gates, limits, assign, weight, offsets, sorted_token};
  const size_t E = c.num_experts, Tk = (size_t)T * c.top_k;
  const size_t bytes[7] = {Tk * 4, Tk * 4, E * 4, (size_t)T * 4, (size_t)T * 4, (E + 1) * 4, (size_t)T * 4};
  for (int i = 0; i < 7; ++i)
    if (misaligned(bufs[i], 4)) return fail(AFD_EINVAL, "capacity routing buffers must be 4-byte aligned");
  for (int i = 0; i < 7; ++i)
    for (int j = i + 1; j < 7; ++j)
      if (bufs[i] && bufs[j] && bytes[i] && bytes[j] && overlaps(bufs[i], bytes[i], bufs[j], bytes[j]))
        return fail(AFD_EINVAL, "capacity routing buffers overlap");
  hipError_t e = afd::launch_route_capacity(ids, gates, T, c.num_experts, c.top_k, base_capacity, adaptive ? 1 : 0,
                                            limits, assign, weight, offsets, sorted_token,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "capacity routing launch");
  return AFD_OK;
}

extern "C" int afd_ffn_route_from_capacity(afd_ffn_t h, const int32_t* assign, const float* weight,
                                           const int32_t* offsets, const int32_t* sorted_token, int32_t T,
                                           const afd_route* r, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!offsets) return fail(AFD_EINVAL, "offsets is NULL");
  if (T > 0 && (!assign || !weight || !sorted_token)) return fail(AFD_EINVAL, "assign, weight or sorted_token is NULL");
  if (misaligned(assign, 4) || misaligned(weight, 4) || misaligned(offsets, 4) || misaligned(sorted_token, 4))
    return fail(AFD_EINVAL, "capacity result buffers must be 4-byte aligned");
  const size_t tb = (size_t)T * 4, ob = ((size_t)h->cfg.num_experts + 1) * 4;
  if ((assign && overlaps_route(assign, tb, h, r, T)) || (weight && overlaps_route(weight, tb, h, r, T)) ||
      overlaps_route(offsets, ob, h, r, T) || (sorted_token && overlaps_route(sorted_token, tb, h, r, T)))
    return fail(AFD_EINVAL, "a capacity result buffer overlaps a route buffer");
  hipError_t e = afd::launch_route_from_capacity(assign, weight, offsets, sorted_token, T, h->cfg.num_experts,
                                                 h->cfg.top_k, r->topk_ids, r->topk_gates, r->expert_counts,
                                                 r->expert_offsets, r->sorted_pair, r->pair_pos,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route from capacity launch");
  note_capacity_route(h, r, T);
  return AFD_OK;
}

extern "C" int afd_ffn_route_hidden(afd_ffn_t h, const void* x, const void* w_router, const float* bias,
                                    float* logits, int32_t T, const afd_route* r, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!x || !w_router || !logits) return fail(AFD_EINVAL, "x, w_router or logits is NULL");
  if (misaligned(x, 16) || misaligned(w_router, 16)) return fail(AFD_EINVAL, "x and w_router must be 16-byte aligned");
  if (misaligned(bias, 4) || misaligned(logits, 4)) return fail(AFD_EINVAL, "bias and logits must be 4-byte aligned");
  if (T == 0) return AFD_OK;
  {
    const afd_ffn_config& c = h->cfg;
    const size_t a = c.dtype == AFD_F32 ? 4 : 2;
    const size_t lb = (size_t)T * c.num_experts * 4;
    if (overlaps(logits, lb, x, (size_t)T * c.hidden * a) ||
        overlaps(logits, lb, w_router, (size_t)c.num_experts * c.hidden * a))
      return fail(AFD_EINVAL, "logits overlaps x or w_router");
    if (overlaps_route(logits, lb, h, r, T)) return fail(AFD_EINVAL, "logits overlap a route buffer");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const afd_ffn_config& c = h->cfg;
  {
    StageScope s(h, st, AFD_STAGE_ROUTER_PROJ);
    hipError_t e = afd::launch_router_proj(x, w_router, bias, T, c.hidden, c.num_experts, c.dtype == AFD_F32,
                                           logits, st);
    if (e != hipSuccess) return hip_fail(e, "router projection launch");
    s.done();
  }
  return afd_ffn_route(h, logits, T, r, stream);
}

static afd_workspace handle_workspace(const afd_ffn* h) {
  return {h->h_routed, h->h_shared, h->o_routed, h->o_shared, h->xq,        h->xs,
          h->hq_routed, h->hs_routed, h->hq_shared, h->hs_shared, h->fused_sync};
}

// Steps a0 and a5-a8 on checked arguments.  fp8 layers: x (bf16) is quantised here,
// or, when x is NULL, xq / xs are the caller's e4m3 codes and scales of it.
static int forward_checked(afd_ffn_t h, const afd_workspace& ws, const void* x, const uint8_t* xq, const float* xs,
                           int32_t T, const afd_route* r, void* y, hipStream_t st) {
  const afd_ffn_config& c = h->cfg;
  const int H = c.hidden, M = c.inter, Ms = c.shared_inter, E = c.num_experts, k = c.top_k;
  const int P = T * k;
  const bool f32 = c.dtype == AFD_F32;
  const bool fp8 = c.dtype == AFD_FP8_E4M3;

  afd::GroupedGemm g1 = {};
  g1.counts = r->expert_counts;
  g1.offsets = r->expert_offsets;
  g1.sorted_pair = r->sorted_pair;
  g1.E = E;
  g1.k = k;
  g1.gather_routed = 1;
  g1.shared_rows = Ms > 0 ? T : 0;
  g1.K_routed = H;
  g1.K_shared = H;
  g1.groups_routed = M / 16;
  g1.groups_shared = Ms / 16;
  g1.w_routed = h->w_gu;
  g1.w_expert_elems = h->w_gu_expert_elems;
  g1.w_shared = h->ws_gu;
  g1.a_routed = x;
  g1.a_shared = x;
  g1.lda_routed = H;
  g1.lda_shared = H;
  g1.out_routed = ws.h_routed;
  g1.out_shared = ws.h_shared;
  g1.ldo_routed = M;
  g1.ldo_shared = Ms;

  afd::GroupedGemm g2 = g1;
  g2.gather_routed = 0;
  g2.K_routed = M;
  g2.K_shared = Ms;
  g2.groups_routed = H / afd::kGroupCols;
  g2.groups_shared = H / afd::kGroupCols;
  g2.w_routed = h->w_d;
  g2.w_expert_elems = h->w_d_expert_elems;
  g2.w_shared = h->ws_d;
  g2.a_routed = ws.h_routed;
  g2.a_shared = ws.h_shared;
  g2.lda_routed = M;
  g2.lda_shared = Ms;
  g2.out_routed = ws.o_routed;
  g2.out_shared = ws.o_shared;
  g2.ldo_routed = H;
  g2.ldo_shared = H;

  if (fp8) {
    g1.a_routed = x ? ws.xq : xq;
    g1.a_shared = g1.a_routed;
    g1.as_routed = x ? ws.xs : xs;
    g1.as_shared = g1.as_routed;
    g1.s_routed = h->s_gu;
    g1.s_expert_elems = (size_t)(H / 128) * (2 * M / 128);
    g1.s_shared = h->ss_gu;
    g2.a_routed = ws.hq_routed;
    g2.a_shared = ws.hq_shared;
    g2.as_routed = ws.hs_routed;
    g2.as_shared = ws.hs_shared;
    g2.s_routed = h->s_d;
    g2.s_expert_elems = (size_t)(M / 128) * (H / 128);
    g2.s_shared = h->ss_d;
    return forward_fp8(h, ws, x, T, r, y, st, g1, g2);
  }

  // Few rows per expert (decode batches): 16-row weight-streaming tiles.  Many rows:
  // 128-row tiles, so each expert's weights are read once per 128 of its rows.
  const bool tiled = !f32 && use_tiled(h, route_rows(h, r, T));
  if (!f32 && !tiled && h->gemm_mode == AFD_GEMM_FUSED && H % 256 == 0 && M % 256 == 0 && Ms % 256 == 0 &&
      h->fused_blocks > 0 && ws.fused_sync) {
    // both GEMMs in one persistent launch; the down epilogue applies the gates
    {
      StageScope s(h, st, AFD_STAGE_FUSED);
      hipError_t e = afd::launch_gemm_bf16_fused(g1, g2, r->topk_gates, ws.fused_sync,
                                                 reinterpret_cast<int*>(ws.fused_sync + 2), h->fused_blocks,
                                                 h->fused_spin_limit, st);
      if (e != hipSuccess) return hip_fail(e, "fused gate/up + down launch");
      s.done();
    }
    StageScope s(h, st, AFD_STAGE_COMBINE);
    hipError_t e = afd::launch_combine(ws.o_routed, Ms ? ws.o_shared : nullptr, r->topk_gates, r->pair_pos, T, k, H, y,
                                       true, st, true);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    s.done();
    return AFD_OK;
  }
  long long items1, items2;
  if (tiled) {
    const int tr = afd::tiled_rows(), tg = afd::tiled_groups();
    items1 = afd::grouped_items_bound(P, E, (g1.groups_routed + tg - 1) / tg, g1.shared_rows,
                                      (g1.groups_shared + tg - 1) / tg, tr);
    items2 = afd::grouped_items_bound(P, E, (g2.groups_routed + tg - 1) / tg, g2.shared_rows,
                                      (g2.groups_shared + tg - 1) / tg, tr);
  } else {
    items1 = afd::grouped_items_bound(P, E, g1.groups_routed, g1.shared_rows, g1.groups_shared, afd::kTileRows);
    items2 = afd::grouped_items_bound(P, E, g2.groups_routed, g2.shared_rows, g2.groups_shared, afd::kTileRows);
  }
  {
    StageScope s(h, st, AFD_STAGE_GATE_UP);
    hipError_t e = f32     ? afd::launch_gemm_f32(g1, true, items1, h->gemm_blocks[2], st)
                   : tiled ? afd::launch_gemm_bf16_tiled(g1, true, items1, h->num_cus, st)
                           : afd::launch_gemm_bf16(g1, true, items1, h->gemm_blocks[0], st);
    if (e != hipSuccess) return hip_fail(e, "gate/up GEMM launch");
    s.done();
  }
  {
    StageScope s(h, st, AFD_STAGE_DOWN);
    hipError_t e = f32     ? afd::launch_gemm_f32(g2, false, items2, h->gemm_blocks[3], st)
                   : tiled ? afd::launch_gemm_bf16_tiled(g2, false, items2, h->num_cus, st)
                           : afd::launch_gemm_bf16(g2, false, items2, h->gemm_blocks[1], st);
    if (e != hipSuccess) return hip_fail(e, "down GEMM launch");
    s.done();
  }
  {
    StageScope s(h, st, AFD_STAGE_COMBINE);
    hipError_t e = afd::launch_combine(ws.o_routed, Ms ? ws.o_shared : nullptr, r->topk_gates, r->pair_pos, T, k, H, y,
                                       !f32, st);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    s.done();
  }
  return AFD_OK;
}

extern "C" int afd_ffn_forward(afd_ffn_t h, const void* x, int32_t T, const afd_route* r, void* y, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!x || !y) return fail(AFD_EINVAL, "x or y is NULL");
  if (misaligned(x, 16) || misaligned(y, 16)) return fail(AFD_EINVAL, "x and y must be 16-byte aligned");
  if (T == 0) return AFD_OK;
  const size_t rowb = (size_t)h->cfg.hidden * (h->cfg.dtype == AFD_F32 ? 4 : 2);
  if (overlaps(x, (size_t)T * rowb, y, (size_t)T * rowb)) return fail(AFD_EINVAL, "x and y overlap");
  if (overlaps_route(y, (size_t)T * rowb, h, r, T)) return fail(AFD_EINVAL, "y overlaps a route buffer");
  return forward_checked(h, handle_workspace(h), x, nullptr, nullptr, T, r, y, static_cast<hipStream_t>(stream));
}

// The intermediate buffers of a forward over T tokens carved from `base` (256-byte
// aligned pieces, in the sizes the handle's workspace has for max_tokens); returns the
// bytes needed.  base == NULL: only the size.
static size_t carve_workspace(const afd_ffn_config& c, size_t T, unsigned char* base, afd_workspace* ws) {
  const size_t H = c.hidden, M = c.inter, Ms = c.shared_inter, P = T * c.top_k;
  const bool fp8 = c.dtype == AFD_FP8_E4M3;
  const size_t hes = c.dtype == AFD_BF16 ? 2 : 4, oes = c.dtype == AFD_F32 ? 4 : 2;
  // the fused decode launch's barrier counters come first: the array is zero at load
  // and every launch leaves them at zero
  const size_t bytes[11] = {256, P * M * hes,   T * Ms * hes,  P * H * oes,   Ms ? T * H * oes : 0,
                            fp8 ? T * H : 0, fp8 ? T * (H / 128) * 4 : 0, fp8 ? P * M : 0,
                            fp8 ? P * (M / 128) * 4 : 0, fp8 ? T * Ms : 0, fp8 ? T * (Ms / 128) * 4 : 0};
  void** dst[11] = {(void**)&ws->fused_sync, &ws->h_routed, &ws->h_shared, &ws->o_routed, &ws->o_shared,
                    (void**)&ws->xq, (void**)&ws->xs, (void**)&ws->hq_routed, (void**)&ws->hs_routed,
                    (void**)&ws->hq_shared, (void**)&ws->hs_shared};
  size_t off = 0;
  for (int i = 0; i < 11; ++i) {
    if (base) *dst[i] = bytes[i] ? base + off : nullptr;
    off += (bytes[i] + 255) / 256 * 256;
  }
  return off;
}

extern "C" int afd_ffn_forward_noalloc(afd_ffn_t h, const void* x, int32_t T, const afd_route* r, void* y,
                                       void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (!x || !y) return fail(AFD_EINVAL, "x or y is NULL");
  if (misaligned(x, 16) || misaligned(y, 16)) return fail(AFD_EINVAL, "x and y must be 16-byte aligned");
  if (T == 0) return AFD_OK;
  const size_t rowb = (size_t)h->cfg.hidden * (h->cfg.dtype == AFD_F32 ? 4 : 2);
  if (overlaps(x, (size_t)T * rowb, y, (size_t)T * rowb)) return fail(AFD_EINVAL, "x and y overlap");
  if (overlaps_route(y, (size_t)T * rowb, h, r, T)) return fail(AFD_EINVAL, "y overlaps a route buffer");
  // The buffers are laid out for the handle's max_tokens, as its own workspace is: any
  // route the handle accepts (at most max_tokens * top_k rows) then stays inside them.
  afd_workspace ws = {};
  const size_t need = carve_workspace(h->cfg, (size_t)h->cfg.max_tokens, nullptr, &ws);
  if (need > kScratchBytes)
    return fail(AFD_EINVAL, "max_tokens=%d needs %zu bytes of intermediate buffers, above the %zu-byte static scratch",
                h->cfg.max_tokens, need, kScratchBytes);
  void* base = h->device >= 0 && h->device < kMaxDevices ? g_scratch[h->device] : nullptr;
  if (!base) return fail(AFD_EHIP, "no scratch address for device %d", h->device);
  carve_workspace(h->cfg, (size_t)h->cfg.max_tokens, static_cast<unsigned char*>(base), &ws);
  return forward_checked(h, ws, x, nullptr, nullptr, T, r, y, static_cast<hipStream_t>(stream));
}

extern "C" int afd_ffn_forward_fp8_input(afd_ffn_t h, const uint8_t* xq, const float* xs, int32_t T,
                                         const afd_route* r, void* y, void* stream) {
  int rc = check_route(h, r, T);
  if (rc) return rc;
  if (h->cfg.dtype != AFD_FP8_E4M3) return fail(AFD_EUNSUPPORTED, "pre-quantised input needs an fp8 layer");
  if (!xq || !xs || !y) return fail(AFD_EINVAL, "xq, xs or y is NULL");
  if (misaligned(xq, 16) || misaligned(y, 16) || misaligned(xs, 4))
    return fail(AFD_EINVAL, "xq and y must be 16-byte aligned, xs 4-byte aligned");
  if (T == 0) return AFD_OK;
  const size_t H = h->cfg.hidden, yb = (size_t)T * H * 2, qb = (size_t)T * H, sb = (size_t)T * (H / 128) * 4;
  if (overlaps(xq, qb, y, yb) || overlaps(xs, sb, y, yb) || overlaps(xq, qb, xs, sb))
    return fail(AFD_EINVAL, "xq, xs and y overlap");
  if (overlaps_route(y, yb, h, r, T)) return fail(AFD_EINVAL, "y overlaps a route buffer");
  return forward_checked(h, handle_workspace(h), nullptr, xq, xs, T, r, y, static_cast<hipStream_t>(stream));
}

extern "C" int afd_ffn_set_gemm_kernel(afd_ffn_t h, int kernel) {
  if (!h) return fail(AFD_EINVAL, "handle is NULL");
  if (kernel < AFD_GEMM_AUTO || kernel > AFD_GEMM_FUSED) return fail(AFD_EINVAL, "unknown GEMM kernel %d", kernel);
  h->gemm_mode = kernel;
  return AFD_OK;
}

extern "C" int afd_ffn_set_profiling(afd_ffn_t h, int on) {
  if (!h) return fail(AFD_EINVAL, "handle is NULL");
  h->profiling = on != 0;
  return AFD_OK;
}

extern "C" int afd_ffn_profile_read(afd_ffn_t h, double* ms, int64_t* launches, int n_stages) {
  if (!h) return fail(AFD_EINVAL, "handle is NULL");
  if (n_stages < 0 || (n_stages > 0 && (!ms || !launches))) return fail(AFD_EINVAL, "bad output arrays");
  for (int i = 0; i < n_stages; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  if (h->ev_used > 0) {
    hipError_t e = hipEventSynchronize(h->ev_pool[h->ev_used - 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  for (size_t i = 0; i < h->ev_stage.size(); ++i) {
    float t = 0.f;
    hipError_t e = hipEventElapsedTime(&t, h->ev_pool[2 * i], h->ev_pool[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    const int s = h->ev_stage[i];
    if (s < n_stages) {
      ms[s] += t;
      launches[s] += 1;
    }
  }
  h->ev_stage.clear();
  h->ev_used = 0;
  return AFD_OK;
}
