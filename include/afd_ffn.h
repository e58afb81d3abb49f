/*
 * afd_ffn.h -- C ABI of the MI355X (gfx950) MoE expert-FFN layer: the compute an
 * FFN instance runs under Attention-FFN disaggregation.
 *
 * The operation.  The FFN service of a disaggregated deployment has no scheduler,
 * no API traffic and no KV cache; per step it receives a batch of hidden states,
 * runs gate routing plus expert computation, and returns the layer output
 * ("大模型推理的内存与计算解耦：AFD 架构解析与性能验证", §3, the FFN service and
 * the data-flow loop of one decode iteration).  For T tokens x[T,H] with fp32
 * router logits[T,E]:
 *
 *   route   : per token, the top_k experts with the largest logits (ties to the
 *             lower expert index) and gates = their softmax probabilities
 *             renormalised to sum to 1 (the router of "MoE 大规模分布式推理工程实战：
 *             从 All-to-All 通信到动态专家放置", §4.1, which normalises the selected
 *             logits with a softmax);
 *             then the (token, slot) pairs are sorted by expert with per-expert
 *             counts, an exclusive prefix sum and a placement pass (the count /
 *             prefix-offset / pack steps of the same page's §2.2; the pre-sorting of
 *             routed tokens that the omica.com.cn AFD article's §3.3 recommends);
 *   forward : per pair (t, e): h = SiLU(x_t Wgu[e][:, :M]) * (x_t Wgu[e][:, M:]),
 *             o = h Wd[e]; y_t = sum_j gate_tj o_tj in slot order, plus a shared
 *             expert's output with gate 1 when the layer has one.  6*H*M FLOPs per
 *             pair (the omica.com.cn AFD article, §2.1).
 *
 * Data types (afd_ffn_config.dtype):
 *   AFD_F32      x, weights and y are float32.
 *   AFD_BF16     x, weights and y are bfloat16.
 *   AFD_FP8_E4M3 weights are OCP e4m3 codes with one float32 scale per 128x128
 *                block; x and y are bfloat16; x and h are quantised to e4m3 per
 *                token and per 128 channels (scale amax/448) inside forward (the
 *                FP8/BF16 mixed precision of the omica.com.cn AFD article, §3.3).
 * All accumulation is float32.  In the bf16 and fp8 layers each expert's output
 * row o_tj is rounded to bf16 before the combine (which sums in float32 and rounds
 * y once); the fp32 layer keeps o_tj in float32.
 *
 * Memory.  Every pointer argument is a device pointer (HIP, same device as the
 * handle), except `cfg`, `out` and the route struct itself, which are host
 * pointers.  Row-major layouts throughout.  Alignment (checked: AFD_EINVAL): the
 * weights, x, y, w_router, the fp8 codes xq and the quantiser's source 16 bytes, the
 * quantiser's codes 8 bytes, every other buffer 4 bytes.  Buffers a call writes must
 * not overlap the ones it reads or the route buffers (checked: AFD_EINVAL), nor may the
 * route buffers overlap each other.  The caller owns all buffers it passes;
 * the library never frees them.  afd_ffn_create copies the weights into a layout
 * of its own (tiles ordered for the matrix cores) and owns that copy and a
 * workspace sized from max_tokens until afd_ffn_destroy; the caller's weight
 * buffers may be freed once create has returned.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default stream).
 * route and forward only enqueue work on it: no host synchronisation, no device
 * read-back and no allocation, so both can be captured in a HIP graph.  A fault
 * in a kernel surfaces at the caller's next synchronisation.  Calls on one handle
 * share its workspace: two forwards in flight at once on different streams race.
 *
 * Errors.  Every int-returning function returns AFD_OK (0) or a negative code;
 * afd_ffn_strerror names the code and afd_ffn_last_error gives the detail of the
 * calling thread's last failure.  Arguments are checked on the host before any
 * work is enqueued; a failed call enqueues nothing.  T = 0 is a successful no-op.
 * Logits must be finite (not checked).
 */
#ifndef AFD_FFN_H_
#define AFD_FFN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFD_OK 0
#define AFD_EINVAL -1       /* a null pointer, a size out of range or misaligned */
#define AFD_EUNSUPPORTED -2 /* a data type or shape this build does not implement */
#define AFD_ENOMEM -3       /* device allocation failed in create */
#define AFD_EHIP -4         /* a HIP runtime call or kernel launch failed */

typedef enum afd_dtype { AFD_F32 = 0, AFD_BF16 = 1, AFD_FP8_E4M3 = 2 } afd_dtype;

/* Layer shape.  hidden, inter and shared_inter must be multiples of 128;
 * 1 <= top_k <= min(num_experts, 32); 1 <= num_experts <= 1024;
 * 1 <= max_tokens and max_tokens * top_k < 2^31; for the fp8 dtype also
 * max_tokens * hidden, max_tokens * top_k * inter and max_tokens * shared_inter
 * below 2^32 (activation matrices under 4 GiB). */
typedef struct afd_ffn_config {
  int32_t hidden;       /* H */
  int32_t inter;        /* M, intermediate size of each routed expert */
  int32_t num_experts;  /* E */
  int32_t top_k;        /* k */
  int32_t max_tokens;   /* largest T any call will pass */
  int32_t shared_inter; /* intermediate size of the always-on shared expert, 0 = none */
  int32_t dtype;        /* afd_dtype */
} afd_ffn_config;

/* Routing result of one batch, in caller-owned device buffers sized for
 * max_tokens (P = T * top_k pairs; pair p = t * top_k + j is slot j of token t). */
typedef struct afd_route {
  int32_t* topk_ids;       /* [max_tokens * k] expert of each pair, slots by rank */
  float* topk_gates;       /* [max_tokens * k] renormalised gates */
  int32_t* expert_counts;  /* [E] pairs routed to each expert */
  int32_t* expert_offsets; /* [E + 1] exclusive prefix sum of counts; [E] = P */
  int32_t* sorted_pair;    /* [max_tokens * k] pair id at each expert-sorted position,
                              ascending token order inside an expert */
  int32_t* pair_pos;       /* [max_tokens * k] inverse: sorted position of each pair */
} afd_route;

typedef struct afd_ffn* afd_ffn_t;

/* Create a layer: the routed experts (and the optional shared expert) of one MoE
 * layer as an FFN instance holds them ("大模型推理的内存与计算解耦：AFD 架构解析与性能
 * 验证", §3; expert shapes of the omica.com.cn AFD article, §2.1).
 * w_gate_up [E, H, 2M] (columns [0, M) gate, [M, 2M) up) and
 * w_down [E, M, H] in the config's dtype.  For AFD_FP8_E4M3, s_gate_up
 * [E, H/128, 2M/128] and s_down [E, M/128, H/128] are the fp32 block scales
 * (weight = code * scale); they must be NULL otherwise.  With shared_inter > 0,
 * ws_gate_up [H, 2*shared_inter] and ws_down [shared_inter, H] (and for fp8
 * ss_gate_up [H/128, 2*shared_inter/128], ss_down [shared_inter/128, H/128]) hold
 * the shared expert; NULL otherwise.  Enqueues the weight repack on `stream` and
 * synchronises it before returning.  On success *out holds the handle. */
int afd_ffn_create(const afd_ffn_config* cfg, const void* w_gate_up, const void* w_down,
                   const float* s_gate_up, const float* s_down, const void* ws_gate_up,
                   const void* ws_down, const float* ss_gate_up, const float* ss_down, void* stream,
                   afd_ffn_t* out);

/* Route T tokens: fp32 logits [T, E] -> every field of *r (see afd_route): the
 * top-k softmax router of "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家
 * 放置" (§4.1) and the count / prefix-offset / pack steps of its §2.2 (the "route"
 * of the operation above).  0 <= T <= max_tokens. */
int afd_ffn_route(afd_ffn_t h, const float* logits, int32_t T, const afd_route* r, void* stream);

/* Route T tokens with a bias that steers only the choice of experts: the dynamic
 * per-expert bias of "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家放置"
 * (§4.1, load balancing by a bias on the router scores, as in DeepSeek-V3's
 * bias-based balancing), in the form where the bias decides which experts a token
 * goes to while the gate weights follow the router's own scores.
 *   key[t, e]  = scores[t, e] + bias[e], rounded to fp32;
 *   ids[t, :]  = the top_k experts by (key descending, expert index ascending);
 *   gates[t, j]= softmax of the unbiased scores of the chosen experts (renormalised
 *                over them, fp32).
 * scores [T, E] and bias [E] are fp32 device buffers (neither may be NULL); every
 * field of *r is filled as by afd_ffn_route, whose result this equals when bias is
 * all zeros.  0 <= T <= max_tokens. */
int afd_ffn_route_select_bias(afd_ffn_t h, const float* scores, const float* bias, int32_t T, const afd_route* r,
                              void* stream);

/* Route T tokens from their hidden states: the router projection of "MoE 大规模分布式
 * 推理工程实战：从 All-to-All 通信到动态专家放置" (§4.1), a bias-free linear map from
 * the hidden size to the experts plus a per-expert dynamic bias, followed by the
 * routing of afd_ffn_route.
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h] + bias[e]   (fp32 accumulation)
 * x [T, H] and w_router [E, H] (row e is expert e's gate vector) are fp32 for AFD_F32
 * and bf16 otherwise; bias [E] is fp32, or NULL for none.  The bias takes part in the
 * selection and in the gates, which are the softmax of the selected biased logits, as
 * in that router.  logits [T, E] fp32 (caller-owned device memory, not overlapping
 * the inputs; checked: AFD_EINVAL) receives the biased logits and is then routed exactly as
 * afd_ffn_route(h, logits, T, r, stream) would route it.  0 <= T <= max_tokens. */
int afd_ffn_route_hidden(afd_ffn_t h, const void* x, const void* w_router, const float* bias, float* logits,
                         int32_t T, const afd_route* r, void* stream);

/* Capacity-aware routing of T tokens: the adaptive token dropper of "MoE 大规模分布式
 * 推理工程实战：从 All-to-All 通信到动态专家放置" (§4.2), for one batch.
 *   ids [T, k] int32 (k = top_k; row t is token t's preference list, most preferred
 *   first, as afd_ffn_route writes r->ids) and gates [T, k] fp32 (r->gates): inputs.
 *   limits [E] int32, read and written: each expert's capacity; when `adaptive` is
 *   non-zero it is updated after the batch (count >= limit: trunc(1.2 limit), at most
 *   INT32_MAX; count < limit / 2: max(base_capacity, trunc(0.9 limit)); else kept).
 *   Limits are expected to be >= 0; start them at base_capacity for a fresh dropper.
 * Counts start at zero for the batch.  Tokens are decided in ascending order: token t
 * goes to the first expert of its list whose count is below its limit, with that
 * slot's gate, and to no other expert; if every listed expert is full, the least-loaded
 * expert (smallest count, lowest index on ties) takes it with half of gates[t, 0] when
 * its count is below 1.5 x its limit; otherwise the token is dropped.  Outputs:
 *   assign [T] int32: the expert, or -1 when dropped;  weight [T] fp32: the gate it
 *   carries (0 when dropped);  offsets [E+1] int32: exclusive prefix sum of the
 *   per-expert counts (offsets[E] = tokens kept);  sorted_token [T] int32: the kept
 *   tokens grouped by expert, in token order within each (entries from offsets[E]
 *   on are not written).
 * All buffers are caller-owned device memory, 4-byte aligned, pairwise disjoint
 * (checked: AFD_EINVAL).  ids values outside [0, E) are never chosen.  T = 0 still
 * writes offsets and adapts the limits.  0 <= T <= min(max_tokens, 2^21),
 * base_capacity >= 0.
 * The decisions are sequential by definition; one workgroup makes them. */
int afd_ffn_route_capacity(afd_ffn_t h, const int32_t* ids, const float* gates, int32_t T, int32_t base_capacity,
                           int32_t adaptive, int32_t* limits, int32_t* assign, float* weight, int32_t* offsets,
                           int32_t* sorted_token, void* stream);

/* Route of a capacity result, for afd_ffn_forward: the expert FFN of the tokens the
 * adaptive token dropper of "MoE 大规模分布式推理工程实战：从 All-to-All 通信到动态专家
 * 放置" (§4.2) kept, each through its one expert, scaled by its weight.
 *   assign [T], weight [T], offsets [E+1], sorted_token [T]: the outputs of
 *   afd_ffn_route_capacity for the same T (device memory, 4-byte aligned, not
 *   overlapping the route buffers; checked: AFD_EINVAL).
 * Fills every field of *r: slot 0 of token t holds assign[t] and weight[t], slots 1..k-1
 * hold id -1 and gate 0, counts/offsets are the kept tokens per expert, sorted_pair
 * lists pair t*k of each kept token in the dropper's order.  afd_ffn_forward on this
 * route then gives y[t] = weight[t] * FFN_assign[t](x[t]) (+ the shared expert), and
 * y[t] = the shared expert's output alone (or 0) for a dropped token: the combine skips
 * slots whose gate is 0.  0 <= T <= max_tokens.  The handle remembers (by the route's
 * sorted_pair buffer, for up to 16 routes) that this route holds at most T rows, and
 * the automatic GEMM choice of a forward on it counts T rows rather than T * k; a
 * later afd_ffn_route* call on the same buffers clears that. */
int afd_ffn_route_from_capacity(afd_ffn_t h, const int32_t* assign, const float* weight, const int32_t* offsets,
                                const int32_t* sorted_token, int32_t T, const afd_route* r, void* stream);

/* Expert FFN of T routed tokens (the "forward" of the operation above: the FFN
 * service's expert computation of "大模型推理的内存与计算解耦：AFD 架构解析与性能验证",
 * §3, SwiGLU experts and gate-weighted combine; fp8 layers quantise x and h as the
 * omica.com.cn AFD article's §3.3 describes): x [T, H] (fp32 for AFD_F32, else bf16)
 * and the result of afd_ffn_route for the same T -> y [T, H] (fp32 for AFD_F32,
 * else bf16).  x and y must not overlap (checked: AFD_EINVAL). */
int afd_ffn_forward(afd_ffn_t h, const void* x, int32_t T, const afd_route* r, void* y, void* stream);

/* Expert FFN of an AFD_FP8_E4M3 layer on activations that arrive already quantised
 * (the attention side sends fp8 activations with per-token, per-128-channel scales,
 * the FP8/BF16 mixed precision of the omica.com.cn AFD article, §3.3, which halves
 * the bytes of the attention-to-FFN transfer).  xq [T, H] e4m3 codes and xs
 * [T, H/128] fp32 scales (activation = code * scale), row-major: the layout
 * afd_ffn_quantize_fp8 writes.  y [T, H] bf16.  Identical to afd_ffn_forward on the
 * bf16 activations those codes and scales were quantised from, without its
 * quantisation launch.  Other layer types: AFD_EUNSUPPORTED.  xq, xs and y must not
 * overlap (checked: AFD_EINVAL). */
int afd_ffn_forward_fp8_input(afd_ffn_t h, const uint8_t* xq, const float* xs, int32_t T, const afd_route* r,
                              void* y, void* stream);

/* afd_ffn_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * and the same result, bit for bit, but the intermediate buffers (h, the expert
 * outputs, the fp8 codes and scales of x and h) come from a static device array of
 * 64 MiB that the library holds on each GPU it runs on (the handle's workspace is not
 * used).  It allocates nothing and needs no zeroed memory.  Calls on one GPU share
 * that array: two calls in flight at once on one GPU, on any handles or streams, race.
 * The buffers are laid out for the handle's max_tokens (so that every route the handle
 * accepts fits them): a handle whose layout exceeds 64 MiB (roughly
 * (max_tokens * top_k) * (M + H) * 2 bytes for a bf16 layer, plus the shared expert's
 * max_tokens * (Ms + H) * 2; about 25 KB per pair at H = 7168, M = 2048 in fp8) is
 * refused with AFD_EINVAL and nothing is enqueued.  Arguments and errors otherwise as
 * afd_ffn_forward. */
int afd_ffn_forward_noalloc(afd_ffn_t h, const void* x, int32_t T, const afd_route* r, void* y, void* stream);

/* Release the handle's weights and workspace (the handle's life cycle; no page
 * defines it).  The caller must have synchronised every stream with work of this
 * handle.  NULL is a no-op. */
int afd_ffn_destroy(afd_ffn_t h);

/* Static description of an error code. */
const char* afd_ffn_strerror(int code);

/* Detail of the calling thread's last failed call ("" if none). */
const char* afd_ffn_last_error(void);

/* Device bytes the handle owns (repacked weights plus workspace). */
size_t afd_ffn_device_bytes(afd_ffn_t h);

/* Device bytes of one set of route buffers for this layer (the six afd_route arrays
 * at their sizes for max_tokens: 4 * (4 * max_tokens * top_k + 2 * num_experts + 1)),
 * for callers that carve them out of one allocation; each array must be 4-byte
 * aligned.  One set per batch in flight.  0 for a NULL handle. */
size_t afd_ffn_route_bytes(afd_ffn_t h);

/* The activation quantisation of the fp8 layer as a stand-alone call: rows x cols
 * activations src (row-major; src_dtype AFD_BF16 or AFD_F32) -> e4m3 codes
 * codes[rows, cols] and fp32 scales scales[rows, cols / 128], per row and per 128
 * channels: scale = amax / 448 (1 for an all-zero group), code = e4m3 nearest to
 * v / scale, ties to even, both divisions IEEE fp32 (the FP8/BF16 mixed precision of
 * the omica.com.cn AFD article, §3.3; the forward call of an fp8 layer quantises x
 * and h this way).  cols must be a multiple of 128.  Asynchronous on `stream`. */
int afd_ffn_quantize_fp8(const void* src, int32_t rows, int32_t cols, int32_t src_dtype, uint8_t* codes,
                         float* scales, void* stream);

/* Choice of grouped-GEMM kernel for bf16 and fp8 layers.  AFD_GEMM_AUTO (the default)
 * uses 16-row weight-streaming tiles while experts average at most 8 (bf16) or 12
 * (fp8) routed rows per batch (T * top_k <= 8 * E, resp. 12 * E) and 128-row tiles
 * above that (the measured crossovers); AFD_GEMM_STREAM and AFD_GEMM_TILED force one
 * kernel (results agree to rounding; a tuning and testing knob).
 * AFD_GEMM_FUSED (bf16 layers whose hidden, inter and shared_inter are multiples of
 * 256; others behave as AFD_GEMM_STREAM) runs both grouped GEMMs of the streaming form
 * in one persistent launch: the single-launch expert kernel of "大模型推理的内存与计算
 * 解耦：AFD 架构解析与性能验证" (§5, MegaMoE) -- gate/up items, the first down weights
 * loaded ahead, a grid-wide barrier, then the down items with each routed row's gate
 * applied in their epilogue (the combine then sums unweighted).  Its workgroups must
 * all be resident at once: the launch uses the device's resident count, and a
 * workgroup that waits at the barrier for longer than ~0.1-1 s gives up and writes NaN
 * into the down-projection rows it owns, so the tokens those rows feed get NaN
 * outputs (a loud failure, no hang); nothing else may occupy the device meanwhile.
 * The environment variable AFD_FUSED_SPIN_LIMIT, read when a handle is created,
 * lowers the number of polls before giving up (0 up to 262144; for failure-injection
 * tests).  fp32 layers always use their own kernel.  Takes effect for later forward
 * calls.  Other values: AFD_EINVAL. */
typedef enum afd_gemm_kernel {
  AFD_GEMM_AUTO = 0,
  AFD_GEMM_STREAM = 1,
  AFD_GEMM_TILED = 2,
  AFD_GEMM_FUSED = 3
} afd_gemm_kernel;
int afd_ffn_set_gemm_kernel(afd_ffn_t h, int kernel);

/* Per-kernel timing, for the per-stage measurement the omica.com.cn AFD article's
 * §4.1 asks for (achieved against expected work per kernel).  With profiling on,
 * route and forward bracket each kernel
 * with HIP events on the launch stream.  afd_ffn_profile_read synchronises on the
 * recorded events, writes the summed milliseconds and launch counts of each stage
 * (index = afd_stage) into ms[n_stages] and launches[n_stages], and clears them.
 * Timing adds an event pair per kernel; leave it off for throughput runs. */
typedef enum afd_stage {
  AFD_STAGE_ROUTER = 0,  /* top-k softmax router (for T <= 64 also the permute: one launch) */
  AFD_STAGE_PERMUTE = 1, /* histogram, prefix scan, scatter (T > 64) */
  AFD_STAGE_QUANT = 2,   /* fp8 quantisation of x and h */
  AFD_STAGE_GATE_UP = 3, /* grouped gate/up GEMM with SwiGLU epilogue */
  AFD_STAGE_DOWN = 4,    /* grouped down-projection GEMM */
  AFD_STAGE_COMBINE = 5, /* gate-weighted combine back to token order */
  AFD_STAGE_ROUTER_PROJ = 6, /* router projection of afd_ffn_route_hidden */
  AFD_STAGE_FUSED = 7,   /* gate/up + down in one launch (AFD_GEMM_FUSED) */
  AFD_NUM_STAGES = 8
} afd_stage;
int afd_ffn_set_profiling(afd_ffn_t h, int on);
int afd_ffn_profile_read(afd_ffn_t h, double* ms, int64_t* launches, int n_stages);

#ifdef __cplusplus
}
#endif

#endif /* AFD_FFN_H_ */
