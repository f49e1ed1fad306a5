/*
 * Plain CPU oracle of one MoE layer's forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU path shares no
 * code with it: no header, no helper, no table.
 *
 * Every function is a direct transcription of the layer's definition as the
 * pages state it, in scalar loops with float64 arithmetic over the exact input
 * values (bf16 inputs are widened exactly; fp32 inputs are read as they are).
 * The router's decisions are taken on fp32 logits, as the GPU takes them, so
 * that both sides can be given the same logits and compared bit for bit.
 *
 * Sources (page titles as printed on the pages):
 *  [P1] "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析"
 *  [P3] "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地"
 *
 * Parity pins (see tests/test_oracle_*.py): brute-force routing and bucket
 * permutation in pure Python, closed-form routing weights, the permute/unpermute
 * identity, a dense all-experts-then-mask reference, textbook SwiGLU closed
 * forms (silu(ln 3) = 0.75 ln 3), invariants (weights sum to 1, counts sum to
 * T*k minus drops).  Agreement with numbers printed on the pages cannot be
 * pinned: the pages print no worked numeric example of the layer.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OpenMP threads the parallel outer loops use */
int oracle_threads(void);

/* storage type of a tensor argument (F64: plain doubles, e.g. dequantised weights) */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* FP8 E4M3 (the OCP "E4M3FN" format: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities, S.1111.111 is NaN, largest finite 448).
 * fp8_decode: the exact value of a code.
 * fp8_encode: the code nearest to x, ties to the even code (the one whose mantissa is even),
 * |x| > 448 saturating to +-448; NaN gives 0x7f.  Written from the format's definition. */
double oracle_fp8_decode(uint8_t code);
uint8_t oracle_fp8_encode(float x);

/* Weight-only FP8 quantisation of a [rows, K] matrix, one scale per row (per output
 * channel of a linear layer's [out, in] weight).  The pages name 8-bit quantisation of expert
 * weights for the serving configuration ([P3] §5.2, "w4afp8": 4-bit weights, FP8
 * activations); reading: FP8 weights with per-row fp32 scales, activations kept in bf16.
 *   amax[r]  = max_k |w[r,k]|;
 *   scale[r] = fp32(amax[r] / 448)  (one correctly rounded fp32 division);
 *   q[r,k]   = fp8_encode(fp32(w[r,k] / scale[r]))  (fp32 division), 0 when scale[r] == 0.
 * The dequantised weight is fp8_decode(q[r,k]) * scale[r]. */
void oracle_quantize_fp8(int64_t rows, int64_t K, int dt, const void* w, uint8_t* q,
                         float* scales);

/* out[r,k] = fp8_decode(q[r,k]) * scales[r], exact in float64. */
void oracle_dequantize_fp8(int64_t rows, int64_t K, const uint8_t* q, const float* scales,
                           double* out);

/* FP4 E2M1 (the OCP microscaling element format: 1 sign, 2 exponent bits with bias 1, 1
 * mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN).
 * fp4_decode: value of a 4-bit code; fp4_encode: the nearest code, ties to the even code,
 * |x| > 6 saturating to +-6. */
double oracle_fp4_decode(uint8_t code);
uint8_t oracle_fp4_encode(float x);

/* MXFP4 weight quantisation (the OCP microscaling format's MXFP4: blocks of 32 consecutive
 * elements along K share one E8M0 scale 2^(s - 127)), a reading of [P3] §5.2's 4-bit expert
 * weights.  Per block: amax = max |w|; if amax == 0 the scale code is 127 (scale 1) and every
 * code 0; else e = floor(log2(amax)), shared = clamp(e - 2, -126, 127) (2 = the largest
 * exponent of E2M1, as the format's rule sets it; the clamp keeps the scale a normal float),
 * scale code = shared + 127, and q = fp4_encode(w / 2^shared) (exact division).  K % 32 == 0.
 * q [rows, K/2]: element 2j in the low nibble of byte j, 2j + 1 in the high nibble;
 * scales [rows, K/32]. */
void oracle_quantize_mxfp4(int64_t rows, int64_t K, int dt, const void* w, uint8_t* q,
                           uint8_t* scales);

/* out[r,k] = fp4_decode(code of (r,k)) * 2^(scales[r, k/32] - 127), exact in float64. */
void oracle_dequantize_mxfp4(int64_t rows, int64_t K, const uint8_t* q, const uint8_t* scales,
                             double* out);

/* MXFP8 activation quantisation (the OCP microscaling format with E4M3 elements: blocks of 32
 * consecutive elements along K share one E8M0 scale 2^(s - 127)), a reading of the FP8
 * activations of [P3] §5.2's "w4afp8" serving configuration.  Per block: amax = max |x|; if
 * amax == 0 the scale code is 127 (scale 1) and every code 0; else e = floor(log2(amax)),
 * shared = clamp(e - 8, -126, 127) (8 = the largest exponent of E4M3, the format's rule;
 * block values in [448, 512) x 2^shared saturate), scale code = shared + 127, and
 * q = fp8_encode(x / 2^shared) (exact division).  K % 32 == 0.  q [rows, K] one code per
 * byte, row-major; scales [rows, K/32]. */
void oracle_quantize_mxfp8(int64_t rows, int64_t K, int dt, const void* x, uint8_t* q,
                           uint8_t* scales);

/* out[r,k] = fp8_decode(q[r,k]) * 2^(scales[r, k/32] - 127), exact in float64. */
void oracle_dequantize_mxfp8(int64_t rows, int64_t K, const uint8_t* q, const uint8_t* scales,
                             double* out);

/* Expert capacity, [P3] §2.1 (router sketch, capacity = tokens / experts x
 * factor), with the top-k factor included: floor(T*k/E*factor) in double. */
int32_t oracle_capacity(int32_t T, int32_t k, int32_t E, double factor);

/* Router gate, [P3] §2.1: a bias-free linear map hidden -> experts.
 * logits[t,e] = fp32( sum_h x[t,h] * wg[e,h] ), summed in float64.
 * x is [T,H], wg is [E,H] (out x in), both of storage type `dt`. */
void oracle_gate(int64_t T, int64_t H, int64_t E, int dt, const void* x, const void* wg,
                 float* logits);

/* how a routing bias enters: added to the logits before the softmax (it changes
 * the selection and the weights), or used to rank the experts only */
enum { ORACLE_BIAS_SOFTMAX = 0, ORACLE_BIAS_SELECT = 1 };

/* Softmax, top-k and renormalisation, [P3] §2.1; [P1] §2 (normalised weights).
 * keys l'[t,e] = logits[t,e] (+ bias[e] as one fp32 add when bias != NULL).
 * ids[t, 0..k-1]: the k experts with the largest key, largest first; equal keys
 * order by lower expert id (+0 and -0 are equal keys).
 * w[t,j]: softmax over all experts taken at ids[t,j]; with renormalize != 0
 * divided by the sum of the k selected probabilities.  The softmax is of the
 * keys (bias_mode ORACLE_BIAS_SOFTMAX, the router sketch's comment: the bias is
 * added to the logits) or of the logits alone (ORACLE_BIAS_SELECT: the bias
 * ranks the experts and nothing else, the aux-free balancing of [P3] §2.1 and
 * §4 read so that the bias steers load without changing the mixing weights).
 * margin[t] (optional): key of the k-th minus key of the (k+1)-th expert in
 * float64, +inf when k == E. */
void oracle_route(int64_t T, int64_t E, int64_t k, const float* logits, const float* bias,
                  int renormalize, int bias_mode, int32_t* ids, double* w, double* margin);

/* Routing load statistics and the next balancing bias.  [P1] §11 names the
 * routing metrics to watch (variance of expert load, drop rate, how hot the
 * hottest expert runs) and [P2] ("上线检查清单" / monitoring table) the token
 * count of every expert and the skew of their distribution.
 * raw[e]: slots (t, j) with ids[t,j] == e (ids outside [0, E) are not counted).
 * ints[0..5]: picks = sum raw, dropped = sum max(0, raw[e] - capacity) (0 when
 *   capacity < 0), max_count, hottest (lowest id with max_count), min_count,
 *   idle (experts with raw == 0).
 * reals[0..4]: mean = picks / E, stddev = sqrt(sum (raw[e] - mean)^2 / E)
 *   (population), cv = stddev / mean, max_over_mean = max_count / mean (both 0
 *   when mean == 0), drop_rate = dropped / picks (0 when picks == 0).
 * bias_next[e] (optional, needs capacity >= 1): [P3] §2.1's aux-free update,
 *   clamp(overflow / capacity, -1, 1) with overflow = raw[e] - capacity, taken
 *   with the sign its comment states (an overloaded expert gets a negative
 *   bias, which lowers its keys): clamp((capacity - raw[e]) / capacity, -1, 1),
 *   computed in float64 and rounded once to fp32. */
void oracle_load_stats(int64_t T, int64_t E, int64_t k, int32_t capacity, const int32_t* ids,
                       int32_t* raw, int64_t* ints, double* reals, float* bias_next);

/* Count, capacity drop, sort and pack, [P1] §8 (count, sort and pack by target
 * expert); [P3] §3.1 (grouping by expert id; per-expert buckets filled in
 * token order).  Assignments of expert e are bucketed in ascending token
 * order; with capacity >= 0 only the first `capacity` of each bucket are kept.
 * raw[e] bucket sizes before the drop, counts[e] kept sizes,
 * offsets[E+1] exclusive prefix sum of counts, row_token[offsets[e] + r] the
 * token of the r-th kept entry of e, pos[t,j] its row or -1 when dropped,
 * dropped[t,j] 1 when dropped.  `active` (optional, [T*k]) marks which slots
 * take part at all; an inactive slot is treated as dropped without counting
 * against capacity.  Returns the number of dropped active slots. */
int64_t oracle_permute(int64_t T, int64_t E, int64_t k, int32_t capacity, const int32_t* ids,
                       const uint8_t* active, int32_t* raw, int32_t* counts, int32_t* offsets,
                       int32_t* row_token, int32_t* pos, uint8_t* dropped);

/* One expert's SwiGLU FFN on M rows, [P1] §1 (FFN(x) = W2 s(W1 x) with an added
 * gate projection) and §2 (input and output of hidden size, inner size I):
 * out[m,:] = W2 ( silu(W1 x_m) * (W3 x_m) ), silu(a) = a / (1 + exp(-a)).
 * xr [M,H] storage `dt_x`; w1, w3 [I,H] and w2 [H,I] storage `dt_w` (ORACLE_F64 for
 * dequantised FP8 weights);
 * out [M,H] float64. */
void oracle_expert_ffn(int64_t M, int64_t H, int64_t I, int dt_x, const void* xr, int dt_w,
                       const void* w1, const void* w3, const void* w2, double* out);

/* The SwiGLU FFN with MXFP8 activations (the "afp8" half of [P3] §5.2's w4afp8): each input
 * row is quantised to MXFP8 along H and dequantised (x'); the gate-up output
 * h = silu(W1 x') * (W3 x') (float64) is rounded once to fp32, quantised to MXFP8 along I and
 * dequantised (h'); out = W2 h'.  Arguments as oracle_expert_ffn; H % 32 == 0, I % 32 == 0. */
void oracle_expert_ffn_a8(int64_t M, int64_t H, int64_t I, int dt_x, const void* xr, int dt_w,
                          const void* w1, const void* w3, const void* w2, double* out);

/* Weighted combine and restore of token order, [P1] §2 (y = sum of g_i E_i(x))
 * and §7 (outputs return to their tokens, weighted by the router).
 * y[t,:] = sum over j ascending with pos[t,j] >= 0 of w[t,j] * yp[pos[t,j],:]
 *          (+ ys[t,:] when ys != NULL, the always-on expert with weight 1). */
void oracle_combine(int64_t T, int64_t H, int64_t k, const double* yp, const int32_t* pos,
                    const double* w, const double* ys, double* y);

/* The whole layer on small inputs: gate, route, permute, per-expert FFN,
 * combine (bias_mode as in oracle_route).  w1, w3 [E,I,H]; w2 [E,H,I]; ws1,
 * ws3 [Is,H], ws2 [H,Is] or NULL (Is = 0).  Optional outputs (NULL to skip): logits, ids, w, pos, counts.
 * Returns the number of dropped slots. */
int64_t oracle_layer(int64_t T, int64_t H, int64_t E, int64_t k, int64_t I, int64_t Is,
                     int32_t capacity, int renormalize, int bias_mode, int dt, const void* x,
                     const void* wg,
                     const float* bias, const void* w1, const void* w3, const void* w2,
                     const void* ws1, const void* ws3, const void* ws2, double* y,
                     float* logits_out, int32_t* ids_out, double* w_out, int32_t* pos_out,
                     int32_t* counts_out);

#ifdef __cplusplus
}
#endif
#endif
