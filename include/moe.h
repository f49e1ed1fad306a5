/*
 * moe.h: C ABI of libmoe.so, the forward pass of one Mixture-of-Experts layer
 * on one AMD Instinct MI355X (gfx950), hand-written in HIP.
 *
 * Sources (cited by page title and section):
 *  [P1] "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析"
 *  [P2] "MoE Expert Parallelism 实战：稀疏大模型推理的通信与负载均衡治理"
 *  [P3] "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地"
 *
 * The layer: a router (bias-free linear gate, softmax, top-k, renormalise),
 * then tokens counted, sorted and packed by expert, then each expert's SwiGLU
 * FFN run as one grouped GEMM over its rows, then the routing-weighted combine
 * back into token order ([P1] §2, §7, §8; [P2] "核心原理" §1; [P3] §2.1).
 * On one GPU the pack step stands in for the expert-parallel all-to-all.
 *
 * Conventions shared by every call:
 *  - Every array pointer is a DEVICE pointer; the caller allocates and owns it.
 *    The library never allocates device memory, and retains no pointer after a
 *    call returns, except the expert cache handle: moe_cache_create allocates
 *    its host bookkeeping and two HIP events, and keeps the caller's pool and
 *    pinned host weights, until moe_cache_destroy.  Scratch memory comes from the caller's
 *    workspace (`ws`, `ws_bytes`), sized by moe_workspace_bytes().
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work and return; outputs are ready when the stream reaches that point.
 *    No call synchronises with the host, except the expert cache's reports:
 *    moe_cache_slots and moe_cache_last_step wait for the cache's last
 *    residency step, and moe_cache_load, moe_layer_forward_cached and
 *    moe_layer_forward_cached_w4a8 do so at their end when given a non-NULL
 *    `info` to fill.
 *  - Device arrays start on 16-byte boundaries (hipMalloc and torch's
 *    allocator give 256): the kernels move rows with 16-byte vector accesses.
 *  - Layouts are row-major and contiguous.  Weights use the [out, in] layout
 *    of a linear layer, so both GEMM operands are contiguous along the
 *    reduction dimension.
 *  - `dtype` (MOE_F32 or MOE_BF16) is the storage type of x, the weights, the
 *    packed rows and y.  Accumulation is always fp32; logits and routing
 *    weights are always fp32; ids, counts, offsets and positions are int32.
 *  - Arguments are checked on the host before anything is launched.  On error
 *    nothing is launched and outputs are untouched, with one exception: the
 *    cached layer learns how many distinct experts a batch needs only on the
 *    device, after its routing; a batch that needs more than the cache has
 *    slots leaves the cache unchanged, its outputs are unspecified, and the
 *    call (with `info`) or a later moe_cache_last_step reports
 *    MOE_ERR_UNSUPPORTED.  No C++ exception crosses the ABI.  T = 0 is a
 *    valid no-op.
 *  - Deterministic: identical inputs give bitwise-identical outputs (no
 *    floating-point atomics; every sum has a fixed order).
 *  - Thread-safe: calls from several threads may run at once.  The library's
 *    global state is set once per device and process (each kernel's LDS size
 *    attribute, the compute-unit count), written with atomics; the exceptions
 *    are an expert cache handle (one thread at a time) and the scratch array
 *    of moe_layer_forward_static (overlapping calls on one device race).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL required pointer, k < 1, k > E, negative size, ... */
  MOE_ERR_UNSUPPORTED = 2, /* a size outside what the kernels handle (see moe_dims_t)   */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than moe_workspace_bytes()               */
  MOE_ERR_HIP = 4          /* a HIP runtime error while enqueuing                       */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Layer dimensions.
 *  T  tokens (>= 0), H hidden size, E routed experts (1..1024), k top-k (1..E),
 *  I  expert intermediate size.  I_shared: 0, or the intermediate size of one
 *  always-on shared expert added to every token with weight 1 ([P1] §3 names
 *  shared experts beside routed ones; the weight is a reading).
 *  capacity: < 0 unlimited; >= 0 the most rows one expert keeps, extra
 *  assignments dropped in token order (see moe_capacity).
 *  renormalize: 1 = divide the k picked probabilities by their sum ([P3]
 *  §2.1); 0 = keep the raw softmax probabilities.
 *  bias_mode (moe_bias_mode_t): how a routing bias, when one is given, enters.
 *  Supported: bf16 needs H % 64 == 0, I % 64 == 0 and I_shared % 64 == 0;
 *  fp32 needs H % 4 == 0.  T * k must fit in int32.  The bf16 kernels address
 *  operands with 32-bit byte offsets, so there the packed rows ((T*k + T) x H
 *  and x max(I, I_shared)), x, the gate weight and one expert's matrix must
 *  each stay below 2^31 bytes; larger sizes return MOE_ERR_UNSUPPORTED. */
typedef struct {
  int32_t T, H, E, k, I;
  int32_t I_shared;
  int32_t capacity;
  int32_t renormalize;
  int32_t dtype;     /* moe_dtype_t */
  int32_t bias_mode; /* moe_bias_mode_t */
} moe_dims_t;

/* The per-expert routing bias of [P3] §2.1 (DeepSeek-V3's auxiliary-loss-free
 * balancing) enters the router in one of two ways:
 *  MOE_BIAS_SOFTMAX: added to the logits before the softmax, so it moves both
 *    the selection and the weights (the reading of the router sketch's comment
 *    that the bias is added to the logits);
 *  MOE_BIAS_SELECT: added to the logits only to rank the experts; the weights
 *    are the softmax of the logits without it, so the bias steers load without
 *    changing how the picked experts are mixed. */
typedef enum { MOE_BIAS_SOFTMAX = 0, MOE_BIAS_SELECT = 1 } moe_bias_mode_t;

/* Load statistics of one routing decision, written by moe_load_stats into
 * device memory.  "Picks" are the (token, slot) pairs whose id is in [0, E). */
typedef struct {
  int32_t picks;       /* sum of the per-expert pick counts                        */
  int32_t dropped;     /* picks beyond an expert's capacity (0 when unlimited)      */
  int32_t max_count;   /* most picks of one expert                                  */
  int32_t hottest;     /* the expert with max_count (the lowest id among equals)    */
  int32_t min_count;   /* fewest picks of one expert                                */
  int32_t idle;        /* experts with no pick                                      */
  float mean;          /* picks / E                                                 */
  float stddev;        /* population standard deviation of the per-expert picks     */
  float cv;            /* stddev / mean (0 when mean == 0)                          */
  float max_over_mean; /* max_count / mean (0 when mean == 0)                       */
  float drop_rate;     /* dropped / picks (0 when picks == 0)                       */
} moe_load_stats_t;

/* Stage boundaries of moe_layer_forward at which events can be recorded. */
enum {
  MOE_EV_START = 0,      /* before the gate                                   */
  MOE_EV_GATE = 1,       /* after the gate GEMM                               */
  MOE_EV_ROUTE = 2,      /* after softmax / top-k / renormalise               */
  MOE_EV_PERMUTE = 3,    /* after count / scan / scatter and the tile maps    */
  MOE_EV_GATE_UP = 4,    /* after the grouped gate-up GEMM (+ SiLU*mul)       */
  MOE_EV_DOWN = 5,       /* after the grouped down GEMM                       */
  MOE_EV_END = 6,        /* after the combine (and a separate shared expert)  */
  MOE_NUM_EVENTS = 7
};

/* Optional debug outputs of moe_layer_forward; any pointer may be NULL.
 * events[i], when non-NULL, is a hipEvent_t the call records on `stream` at
 * stage boundary i (per-stage timing; the caller creates and owns the
 * events). */
typedef struct {
  float* logits;     /* [T,E] gate logits (before the bias)          */
  int32_t* topk_ids; /* [T,k]                                         */
  float* topk_w;     /* [T,k]                                         */
  int32_t* counts;   /* [E]   kept rows per expert                    */
  int32_t* offsets;  /* [E+1] exclusive prefix sum of counts          */
  int32_t* pos;      /* [T,k] packed row of each slot, -1 if dropped  */
  int32_t* n_dropped;/* [1]                                           */
  void* events[MOE_NUM_EVENTS];
} moe_debug_out_t;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int32_t status);

/* Expert capacity, host-side: floor(T * k / E * factor) in double.
 * [P3] §2.1 gives capacity as tokens / experts times a factor (1.25 in
 * training, 2.0 in evaluation); the factor k counts every pick of a token
 * (a reading: without it a top-2 layer could keep only half its picks).
 * Returns -1 when E <= 0 or factor < 0. */
int32_t moe_capacity(int32_t T, int32_t k, int32_t E, double factor);

/* Workspace bytes that any call below needs for `dims` (the maximum over all
 * calls; the same workspace serves each of them).  0 on invalid dims. */
size_t moe_workspace_bytes(const moe_dims_t* dims);

/* Router gate, [P3] §2.1: logits = x * Wg^T, a linear map without bias.
 *  x [T,H] (dtype), wg [E,H] (dtype) -> logits [T,E] fp32.
 *  bf16 runs on MFMA (fp32 accumulate); fp32 on vector FMA. */
moe_status_t moe_gate(const moe_dims_t* dims, const void* x, const void* wg, float* logits,
                      void* stream);

/* Softmax, top-k, renormalisation and capacity drop, [P3] §2.1.
 *  logits [T,E] fp32; bias [E] fp32 or NULL.  The selection keys are
 *  logits + bias (one fp32 add).
 *  topk_ids [T,k]: the k experts with the largest key, largest first; equal
 *  keys (+0 == -0) go to the lower expert id.
 *  topk_w [T,k]: their softmax probabilities, renormalised over the k picks
 *  when dims->renormalize; the softmax is of the keys (MOE_BIAS_SOFTMAX) or
 *  of the logits alone (MOE_BIAS_SELECT).
 *  counts [E] (or NULL): rows each expert keeps after the capacity drop.
 *  dropped [T,k] u8 (or NULL): 1 where the slot was dropped (capacity reached
 *  by earlier tokens of that expert).  n_dropped [1] (or NULL).
 *  A non-NULL counts, dropped or n_dropped needs the workspace. */
moe_status_t moe_route(const moe_dims_t* dims, const float* logits, const float* bias,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, uint8_t* dropped,
                       int32_t* n_dropped, void* ws, size_t ws_bytes, void* stream);

/* Count, exclusive prefix sum and stable scatter into expert-contiguous rows,
 * [P1] §8 (count, sort and pack by target expert); [P3] §3.1 (group by
 * expert id, token order kept inside each expert).
 *  topk_ids [T,k]; dropped [T,k] u8 or NULL (NULL = keep every slot).
 *  offsets [E+1]: offsets[e] is the first packed row of expert e, offsets[E]
 *  the number of kept rows R.
 *  row_token [T*k]: the source token of each packed row (first R valid).
 *  pos [T,k]: the packed row of each slot, -1 if dropped.
 *  x_packed [T*k,H] (dtype) or NULL: rows of x gathered in packed order.
 *  x may be NULL when x_packed is NULL. */
moe_status_t moe_permute(const moe_dims_t* dims, const void* x, const int32_t* topk_ids,
                         const uint8_t* dropped, int32_t* offsets, int32_t* row_token,
                         int32_t* pos, void* x_packed, void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU expert FFN, [P1] §1 (FFN with an added gate projection), §2
 * (hidden size in and out, intermediate size inside) and §8 (one grouped GEMM
 * over the tokens each expert collected).
 *  For each expert e and packed row r in [offsets[e], offsets[e+1]):
 *  y_packed[r] = W2[e] ( silu(W1[e] x_packed[r]) * (W3[e] x_packed[r]) ),
 *  silu(a) = a / (1 + exp(-a)).
 *  x_packed [T*k,H], w1 [E,I,H], w3 [E,I,H], w2 [E,H,I], y_packed [T*k,H]
 *  (all dtype); offsets [E+1] on the device (as moe_permute writes them).
 *  The intermediate activation lives in the workspace (bf16 for bf16).
 *  Rows past offsets[E] are not written. */
moe_status_t moe_expert_ffn(const moe_dims_t* dims, const void* x_packed, const int32_t* offsets,
                            const void* w1, const void* w3, const void* w2, void* y_packed,
                            void* ws, size_t ws_bytes, void* stream);

/* Weighted combine and restore of token order, [P1] §2 and §7; [P2] "核心原理"
 * §1 (outputs merged back into the original token order).
 *  y[t] = sum over j = 0..k-1 with pos[t,j] >= 0 of topk_w[t,j] * y_packed[pos[t,j]]
 *         (+ y_shared[t] when y_shared != NULL),
 *  summed in fp32 in slot order, rounded once to dtype.
 *  y_packed [*,H], pos [T,k], topk_w [T,k], y_shared [T,H] or NULL, y [T,H]. */
moe_status_t moe_combine(const moe_dims_t* dims, const void* y_packed, const int32_t* pos,
                         const float* topk_w, const void* y_shared, void* y, void* stream);

/* Routing load statistics, the routing metrics [P1] §11 names (variance of
 * expert load, drop rate, how hot the hottest expert runs) and the per-expert
 * token counts and skew of [P2]'s monitoring table; with bias_next, also the
 * next value of [P3] §2.1's auxiliary-loss-free balancing bias.
 *  topk_ids [T,k] (as moe_route writes them); ids outside [0, E) are ignored.
 *  raw_counts [E] or NULL: picks of each expert before the capacity.
 *  stats [1] (device): see moe_load_stats_t; dropped uses dims->capacity.
 *  bias_next [E] or NULL: clamp((C - raw[e]) / C, -1, 1) with C =
 *  dims->capacity, computed in fp64 and rounded once: the page's
 *  clamp(overflow / capacity, -1, 1), overflow = picks - capacity, with the
 *  sign its comment states (an overloaded expert gets a negative bias, which
 *  lowers its keys).  Needs dims->capacity >= 1, else MOE_ERR_INVALID_ARG.
 *  Needs the workspace.  Integer outputs are exact; the float statistics are
 *  computed in fp64 with a fixed summation order and rounded once. */
moe_status_t moe_load_stats(const moe_dims_t* dims, const int32_t* topk_ids, int32_t* raw_counts,
                            moe_load_stats_t* stats, float* bias_next, void* ws, size_t ws_bytes,
                            void* stream);

/* FP8 E4M3 weight quantisation, one fp32 scale per row.  [P3] §5.2 serves the
 * experts with low-precision weights (its configuration: 4-bit weights, FP8
 * activations) to cut the bytes a decode step streams; the format here is a
 * reading: E4M3 (OCP: sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite 448, no infinities) with a per-row scale, activations bf16.
 *  w [rows, K] of storage `dtype` (MOE_BF16 or MOE_F32), K % 8 == 0, K > 0.
 *  scales[r] = fp32(max_k |w[r,k]| / 448); q[r,k] = the E4M3 code nearest to
 *  fp32(w[r,k] / scales[r]) (ties to even, saturating at +-448), 0 when the
 *  scale is 0.  The dequantised weight is value(q) * scale.
 *  q [rows, K] u8 and scales [rows] fp32 are device outputs.  For a layer,
 *  quantise w1 and w3 as [E*I, H], w2 as [E*H, I] (and the shared expert's
 *  likewise): one scale per output channel. */
moe_status_t moe_quantize_fp8(int64_t rows, int32_t K, int32_t dtype, const void* w, uint8_t* q,
                              float* scales, void* stream);

/* MXFP4 weight quantisation: E2M1 codes (OCP microscaling: sign, 2 exponent bits
 * with bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0
 * scale 2^(s - 127) per 32 consecutive elements of a row, a reading of [P3]
 * §5.2's 4-bit expert weights (weight-only here; activations stay bf16).
 *  w [rows, K] of storage `dtype` (MOE_BF16 or MOE_F32), rows % 32 == 0 and
 *  K % 128 == 0 (else MOE_ERR_UNSUPPORTED).
 *  Per block of 32: amax = max |w|; 0 gives scale code 127 and codes 0; else
 *  shared = clamp(floor(log2(amax)) - 2, -126, 127), scale code = shared + 127,
 *  and each code the E2M1 value nearest to w / 2^shared (ties to even,
 *  saturating at +-6).
 *  Both outputs are blocked by 32 rows and 128 k, so that what the grouped
 *  GEMM reads for 32 weight rows and 128 k is whole 128-byte lines:
 *  q: rows * K/2 bytes, [rows/32, K/128, 32, 64]: element k of row r in byte
 *  ((r/32) * (K/128) + k/128) * 2048 + (r%32) * 64 + (k%128)/2, the low
 *  nibble for even k;
 *  scales: rows * K/32 bytes, [rows/32, K/128, 32, 4]: the scale of row r,
 *  block b (elements 32b .. 32b+31) at byte
 *  ((r/32) * (K/128) + b/4) * 128 + (r%32) * 4 + b%4.
 *  Quantise w1 and w3 as [E*I, H] and w2 as [E*H, I] (I % 32 == 0 keeps an
 *  expert's codes and scales contiguous, E*I*H/2 and E*I*H/32 bytes). */
moe_status_t moe_quantize_mxfp4(int64_t rows, int32_t K, int32_t dtype, const void* w,
                                uint8_t* q, uint8_t* scales, void* stream);

/* moe_expert_ffn with MXFP4 weights (blocked codes and scales as
 * moe_quantize_mxfp4 writes them for w1/w3 as [E*I, H] and w2 as [E*H, I]).
 * dims->dtype
 * must be MOE_BF16, H and I multiples of 128.  The codes widen, times their
 * block scale, exactly to bf16 for the MFMA.  Every group size runs on the
 * 32-row tiles (the weight-streaming shape). */
moe_status_t moe_expert_ffn_mxfp4(const moe_dims_t* dims, const void* x_packed,
                                  const int32_t* offsets, const uint8_t* w1q, const uint8_t* w1s,
                                  const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                  const uint8_t* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                  void* stream);

/* moe_expert_ffn with FP8 weights: w1q/w3q [E,I,H], w2q [E,H,I] E4M3 codes
 * and their per-row scales w1s/w3s [E*I], w2s [E*H] (as moe_quantize_fp8
 * writes them).  dims->dtype must be MOE_BF16 (x_packed, y_packed bf16).
 *  y_packed[r] = W2' ( silu(W1' x_packed[r]) * (W3' x_packed[r]) ) with
 *  W' = value(q) * scale per row: the codes widen exactly to bf16 for the MFMA
 *  and each output column's fp32 sum is multiplied by its row's scale. */
moe_status_t moe_expert_ffn_fp8(const moe_dims_t* dims, const void* x_packed,
                                const int32_t* offsets, const uint8_t* w1q, const float* w1s,
                                const uint8_t* w3q, const float* w3s, const uint8_t* w2q,
                                const float* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                void* stream);

/* moe_layer_forward with FP8 expert weights (the gate stays bf16): as
 * moe_layer_forward, with each expert weight given as E4M3 codes and per-row
 * scales (moe_quantize_fp8); the shared expert's too when dims->I_shared > 0
 * (ws1q/ws3q [I_shared,H] with ws1s/ws3s [I_shared], ws2q [H,I_shared] with
 * ws2s [H]).  dims->dtype must be MOE_BF16. */
moe_status_t moe_layer_forward_fp8(const moe_dims_t* dims, const void* x, const void* wg,
                                   const float* bias, const uint8_t* w1q, const float* w1s,
                                   const uint8_t* w3q, const float* w3s, const uint8_t* w2q,
                                   const float* w2s, const uint8_t* ws1q, const float* ws1s,
                                   const uint8_t* ws3q, const float* ws3s, const uint8_t* ws2q,
                                   const float* ws2s, void* y, const moe_debug_out_t* dbg,
                                   void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward with MXFP4 expert weights (the gate stays bf16), as
 * moe_layer_forward_fp8 with E8M0 block scales in place of the per-row fp32
 * scales; the shared expert's weights likewise.  dims->dtype must be
 * MOE_BF16; H, I and I_shared multiples of 128. */
moe_status_t moe_layer_forward_mxfp4(const moe_dims_t* dims, const void* x, const void* wg,
                                     const float* bias, const uint8_t* w1q, const uint8_t* w1s,
                                     const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                     const uint8_t* w2s, const uint8_t* ws1q, const uint8_t* ws1s,
                                     const uint8_t* ws3q, const uint8_t* ws3s,
                                     const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                     const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                     void* stream);

/* ---- MXFP8 activations with MXFP4 weights ---------------------------------
 * [P3] §5.2 serves the experts with 4-bit weights and FP8 activations.
 * Reading: the activations use the OCP microscaling MXFP8 format (E4M3
 * elements with one E8M0 scale per 32 consecutive elements of a row), the
 * weights MXFP4 as moe_quantize_mxfp4 writes them, and the products run on
 * CDNA4's block-scaled MFMA, which applies both scales in hardware.  Each
 * expert FFN quantises twice: its input rows (along H) and its SwiGLU
 * activation (along I, after silu(a) * g is formed in fp32). */

/* MXFP8 quantisation: x [rows, K] of storage `dtype` (MOE_BF16 or MOE_F32),
 * K % 32 == 0 and K > 0 (else MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED).
 * Per block of 32: amax = max |x|; 0 gives scale code 127 and codes 0; else
 * shared = clamp(floor(log2(amax)) - 8, -126, 127) (8: the largest E4M3
 * exponent), scale code = shared + 127, and each code the E4M3 value nearest
 * to x / 2^shared (ties to even, saturating at +-448).
 *  q [rows, K] u8 codes and scales [rows, K/32] u8, both row-major device
 *  outputs; the dequantised value is value(q) * 2^(scale - 127). */
moe_status_t moe_quantize_mxfp8(int64_t rows, int32_t K, int32_t dtype, const void* x,
                                uint8_t* q, uint8_t* scales, void* stream);

/* moe_expert_ffn_mxfp4 with MXFP8 activations: x_packed (bf16) is quantised
 * to MXFP8 inside the call, then
 *  y_packed[r] = W2' Q( silu(W1' Q(x_packed[r])) * (W3' Q(x_packed[r])) )
 * with Q the MXFP8 round trip along the row and W' the dequantised MXFP4
 * weights; every product is exact and sums in fp32.  dims->dtype must be
 * MOE_BF16; H and I multiples of 128.  Every group size runs on the 32-row
 * tiles.  The workspace (moe_workspace_bytes) holds the quantised rows. */
moe_status_t moe_expert_ffn_w4a8(const moe_dims_t* dims, const void* x_packed,
                                 const int32_t* offsets, const uint8_t* w1q, const uint8_t* w1s,
                                 const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                 const uint8_t* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                 void* stream);

/* moe_layer_forward_mxfp4 with MXFP8 activations: the gate and the routing
 * run on the bf16 x as in moe_layer_forward; x is quantised to MXFP8 once per
 * token (the expert GEMMs gather its rows), and every expert, the shared one
 * included, computes as moe_expert_ffn_w4a8.  Same arguments and limits as
 * moe_layer_forward_mxfp4.  With debug events, the quantisation of x is timed
 * with the permute step. */
moe_status_t moe_layer_forward_w4a8(const moe_dims_t* dims, const void* x, const void* wg,
                                    const float* bias, const uint8_t* w1q, const uint8_t* w1s,
                                    const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                    const uint8_t* w2s, const uint8_t* ws1q, const uint8_t* ws1s,
                                    const uint8_t* ws3q, const uint8_t* ws3s,
                                    const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                    const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---- Expert cache: experts resident in HBM up to a number of slots ----------
 * [P3] §3.2 keeps a subset of the experts in HBM and loads the others from
 * host memory before a batch needs them, evicting the least recently used
 * resident experts.  Here: a caller-allocated device pool of `slots` expert
 * slots (W1, W3, W2 of one expert each, in the layer's storage type) and a
 * device table expert -> slot, managed by a host-side object.  Residency
 * policy (readings): recency = the last batch that requested an expert (ties:
 * lower id); a batch's own experts are never evicted for it; free slots are
 * taken lowest first; missing experts load in ascending id order; a batch
 * that needs more distinct experts than there are slots changes nothing.
 * Residency is decided on the device (one small kernel, from a host list or
 * from the per-expert row counts a layer's routing left on the device), and a
 * copy kernel reads the missing experts from the host arrays over PCIe into
 * their slots, so the host arrays must be pinned (hipHostMalloc, or torch's
 * pin_memory) and stay alive as long as the cache.  Ordering: a residency
 * step runs on the copy stream after the work enqueued so far on the compute
 * stream (which may still read the slots it refills) and after this cache's
 * earlier steps; the compute stream's later work waits for it.  Nothing waits
 * for the host.  bf16 layers only.  A cache
 * holds the experts either in bf16 (moe_cache_create) or as MXFP4 codes and
 * scales (moe_cache_create_mxfp4: [P3] §5.2 serves with the expert cache and
 * 4-bit experts together; a slot then costs about a quarter of the HBM and of
 * the host -> device bytes).  The object holds host bookkeeping (allocated in
 * moe_cache_create*, freed in moe_cache_destroy) and two HIP events; one object
 * must not be used from two threads at once. */
typedef struct moe_expert_cache moe_expert_cache_t;

/* Outcome of one batch's residency request. */
typedef struct {
  int32_t requested;    /* distinct experts the batch needs      */
  int32_t hits;         /* of those, already resident            */
  int32_t loads;        /* copied from host memory               */
  int32_t evictions;    /* resident experts dropped to make room */
  int64_t bytes_loaded; /* host -> device bytes enqueued         */
} moe_cache_step_t;

/* Device bytes of a pool of `slots` expert slots plus the expert -> slot table
 * (0 on invalid dims or slots < 1). */
size_t moe_cache_pool_bytes(const moe_dims_t* dims, int32_t slots);

/* host_w1/host_w3 [E,I,H], host_w2 [E,H,I] (pinned host memory, dims->dtype,
 * owned by the caller and kept alive as long as the cache; not pinned:
 * MOE_ERR_INVALID_ARG); pool: device memory of at least moe_cache_pool_bytes
 * (slots <= 1024).  Only H, E, I and dtype of dims matter here.  On success
 * *cache receives the new object. */
moe_status_t moe_cache_create(const moe_dims_t* dims, int32_t slots, const void* host_w1,
                              const void* host_w3, const void* host_w2, void* pool,
                              size_t pool_bytes, moe_expert_cache_t** cache);

/* Device bytes of a pool of `slots` MXFP4 expert slots (codes, scales) plus
 * the table (0 on invalid dims, slots < 1, or H, I not multiples of 128). */
size_t moe_cache_pool_bytes_mxfp4(const moe_dims_t* dims, int32_t slots);

/* An expert cache of MXFP4 experts: host_w1q/host_w1s and host_w3q/host_w3s
 * as moe_quantize_mxfp4 writes [E*I, H], host_w2q/host_w2s as it writes
 * [E*H, I] (host memory, pinned for asynchronous copies, owned by the caller
 * and kept alive as long as the cache); pool: device memory of at least
 * moe_cache_pool_bytes_mxfp4.  dims->dtype must be MOE_BF16 and H, I
 * multiples of 128 (else MOE_ERR_UNSUPPORTED).  Used by
 * moe_layer_forward_cached_w4a8; moe_cache_load and moe_cache_slots work on
 * it as on a bf16 cache (bytes_loaded counts codes and scales). */
moe_status_t moe_cache_create_mxfp4(const moe_dims_t* dims, int32_t slots,
                                    const uint8_t* host_w1q, const uint8_t* host_w1s,
                                    const uint8_t* host_w3q, const uint8_t* host_w3s,
                                    const uint8_t* host_w2q, const uint8_t* host_w2s, void* pool,
                                    size_t pool_bytes, moe_expert_cache_t** cache);
void moe_cache_destroy(moe_expert_cache_t* cache);

/* Make the n experts in `experts` (host array, ids in [0, E), duplicates
 * allowed) resident: enqueue the residency step and the copies on
 * copy_stream, and make stream wait for them (a prefetch ahead of the batch
 * that needs them).  More distinct experts than slots: MOE_ERR_UNSUPPORTED,
 * nothing enqueued.  info (host) may be NULL; if given, the call waits for
 * the step and reports it. */
moe_status_t moe_cache_load(moe_expert_cache_t* cache, const int32_t* experts, int32_t n,
                            void* copy_stream, void* stream, moe_cache_step_t* info);

/* Host copy of the expert -> slot table (-1: not resident), slot_of [E];
 * waits for the cache's last residency step. */
moe_status_t moe_cache_slots(const moe_expert_cache_t* cache, int32_t* slot_of);

/* The cache's last residency step (moe_cache_load or a cached layer): waits
 * for it and fills info; MOE_ERR_UNSUPPORTED if that batch needed more
 * distinct experts than slots (the cache was left unchanged). */
moe_status_t moe_cache_last_step(const moe_expert_cache_t* cache, moe_cache_step_t* info);

/* moe_layer_forward with the routed experts' weights in an expert cache: after
 * the gate, route and permute, the experts with kept rows are made resident
 * by a residency step on copy_stream (decided on the device from the
 * per-expert row counts; no host round trip), and the grouped GEMMs read each
 * expert's weights from its slot.  The shared expert (dims->I_shared > 0) is
 * given as in moe_layer_forward and is not cached.  The output is bit for bit
 * that of moe_layer_forward with the same weights.  info (host) may be NULL;
 * if given, the call waits for the layer's residency step at its end and
 * reports it.  A batch that needs more distinct experts than the cache has
 * slots leaves the cache unchanged and the output unspecified, reported as
 * MOE_ERR_UNSUPPORTED by this call (with info) or by moe_cache_last_step
 * (slots >= min(E, T*k) rules it out). */
moe_status_t moe_layer_forward_cached(const moe_dims_t* dims, const void* x, const void* wg,
                                      const float* bias, moe_expert_cache_t* cache,
                                      const void* ws1, const void* ws3, const void* ws2, void* y,
                                      const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                      void* stream, void* copy_stream, moe_cache_step_t* info);

/* moe_layer_forward_cached on an MXFP4 expert cache (moe_cache_create_mxfp4),
 * computing as moe_layer_forward_w4a8: MXFP8 activations on the cached MXFP4
 * experts; the shared expert's MXFP4 weights (ws1q/ws1s, ... as in
 * moe_layer_forward_w4a8) are not cached.  The output is bit for bit that of
 * moe_layer_forward_w4a8 with the same codes and scales.  A bf16 cache, or an
 * MXFP4 cache passed to moe_layer_forward_cached, is MOE_ERR_INVALID_ARG.
 * Same waits and failure modes as moe_layer_forward_cached. */
moe_status_t moe_layer_forward_cached_w4a8(const moe_dims_t* dims, const void* x, const void* wg,
                                           const float* bias, moe_expert_cache_t* cache,
                                           const uint8_t* ws1q, const uint8_t* ws1s,
                                           const uint8_t* ws3q, const uint8_t* ws3s,
                                           const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                           const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                           void* stream, void* copy_stream,
                                           moe_cache_step_t* info);

/* The whole layer in one enqueue: gate, route (+bias, capacity), permute,
 * grouped gate-up with SiLU*mul, grouped down, combine.  The pack is fused into
 * the gate-up GEMM's row loads.  The shared expert (dims->I_shared > 0) runs
 * as one more group over all T tokens.
 *  x [T,H], wg [E,H], bias [E] fp32 or NULL (entering as dims->bias_mode
 *  says), w1/w3 [E,I,H], w2 [E,H,I],
 *  ws1/ws3 [I_shared,H], ws2 [H,I_shared] (NULL when I_shared == 0), y [T,H].
 *  dbg: NULL, or a struct whose non-NULL members receive intermediates. */
moe_status_t moe_layer_forward(const moe_dims_t* dims, const void* x, const void* wg,
                               const float* bias, const void* w1, const void* w3, const void* w2,
                               const void* ws1, const void* ws3, const void* ws2, void* y,
                               const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                               void* stream);

/* ---- For callers that cannot allocate ---------------------------------------
 * Code under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc cannot hand the layer a workspace they allocate per call.
 * moe_layer_forward_static is moe_layer_forward (same arguments, same kernels,
 * bit-identical results) without the `ws` / `ws_bytes` pair: its scratch is a
 * device array that the library owns, MOE_STATIC_SCRATCH_MIB MiB per device,
 * allocated with the code object when the library loads on a device and held
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).
 *  - dims whose moe_workspace_bytes() exceeds moe_static_scratch_bytes()
 *    return MOE_ERR_WORKSPACE before anything is launched.  64 MiB holds, for
 *    example, a decode step of 256 tokens with hidden size 7168, 256 routed
 *    experts of width 2048, top-8, and a shared expert of width 2048.
 *  - The array holds the last call's intermediates.  Nothing in it needs to
 *    start at zero: every kernel writes the scratch it later reads.
 *  - Every call on a device shares that device's array: calls that overlap on
 *    one device (different streams, or different threads) race and give
 *    undefined results; calls on one stream are ordered and safe.
 * The first call on a device looks the array's address up (hipGetSymbolAddress)
 * and keeps it; later calls only enqueue. */
#define MOE_STATIC_SCRATCH_MIB 64
size_t moe_static_scratch_bytes(void);
moe_status_t moe_layer_forward_static(const moe_dims_t* dims, const void* x, const void* wg,
                                      const float* bias, const void* w1, const void* w3,
                                      const void* w2, const void* ws1, const void* ws3,
                                      const void* ws2, void* y, const moe_debug_out_t* dbg,
                                      void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
