// Router tail: softmax, top-k selection and renormalisation, one wavefront per token.
//
// Follows the router of "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地"
// §2.1 (softmax over the gate logits, top-k, division by the sum of the picked
// probabilities) and the top-2 example with normalised weights of
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §2.
//
// Selection is taken on the fp32 keys (logit + bias), which orders experts
// exactly as the probabilities do (softmax is monotone), without letting an
// exp rounding merge two distinct keys.  Order: key descending, expert id
// ascending among equal keys, with +0 and -0 equal.  Each lane keeps EPL keys
// in registers; k rounds of a wavefront max over a 64-bit (key, ~id) word pick
// the experts in slot order.
//
// The bias of the same §2.1 (auxiliary-loss-free balancing) either sits inside
// the softmax (the weights are those of the keys) or only ranks the experts
// (the weights are those of the bare logits, so it steers load without
// changing how the picked experts are mixed).
#include "common.hpp"

namespace moe {

// order-preserving map of a float to uint32 (-0 folded onto +0)
__device__ __forceinline__ uint32_t sortable(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  // butterfly: every lane ends with the same, order-fixed sum
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

constexpr int kRouteMaxSplits = 16;  // the most partial sums a split gate leaves

// With gpart != null the logits are the sum of a split gate's S partials (part 0, then 1 .. S - 1:
// the order of the split-K reduction, so the same bits), written to logits_out on the way.
template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int renormalize, int sel_only,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w,
                                                    const float* __restrict__ gpart, int S,
                                                    float* __restrict__ logits_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // whole wavefront leaves together
  const int64_t row0 = (int64_t)t * E, n = (int64_t)T * E;

  // key: what the experts are ranked by; val: what the softmax is taken of
  float key[EPL], val[EPL];
  bool taken[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int e = s * kWave + lane;
    float v = -INFINITY, l = -INFINITY;
    if (e < E) {
      if (gpart) {
        // every partial's load goes out before the first add
        float pv[kRouteMaxSplits];
#pragma unroll
        for (int q = 0; q < kRouteMaxSplits; ++q) pv[q] = q < S ? gpart[q * n + row0 + e] : 0.f;
        l = pv[0];
#pragma unroll
        for (int q = 1; q < kRouteMaxSplits; ++q)
          if (q < S) l += pv[q];
        logits_out[row0 + e] = l;
      } else {
        l = logits[row0 + e];
      }
      v = bias ? l + bias[e] : l;  // one fp32 add
    }
    key[s] = v;
    val[s] = sel_only ? l : v;
    taken[s] = e >= E;
  }

  // slot j's id and key live in lane j % 64, register j / 64
  float selv[EPL];
  int32_t seli[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    selv[s] = 0.f;
    seli[s] = 0;
  }
  float top = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      if (!taken[s]) {
        const uint32_t e = (uint32_t)(s * kWave + lane);
        const uint64_t cand = ((uint64_t)sortable(key[s]) << 32) | (uint32_t)(~e);
        best = cand > best ? cand : best;
      }
    }
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    // the owner lane marks it and reports its softmax value
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      if (s * kWave + lane == e) {
        taken[s] = true;
        v = val[s];
      }
    }
    v = __shfl(v, e & (kWave - 1), kWave);
    if (j == 0) top = v;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      if (s * kWave + lane == j) {
        selv[s] = v;
        seli[s] = e;
      }
    }
  }

  // the shift of the exponentials: the first pick's value is the largest of the row when the
  // softmax is of the keys; of the bare logits, take the picked maximum (renormalised) or the
  // row maximum (raw probabilities), so that the largest term is exp(0)
  if (sel_only) {
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      const int i = s * kWave + lane;
      if (renormalize ? i < k : i < E) m = fmaxf(m, renormalize ? selv[s] : val[s]);
    }
    top = wave_max_f32(m);
  }
  // weights: exp(value - shift) over the picked experts, divided by the picked sum
  // (renormalised) or by the sum over every expert (raw softmax probability)
  float ex[EPL];
  float part = 0.f;
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int j = s * kWave + lane;
    ex[s] = j < k ? expf(selv[s] - top) : 0.f;
  }
  if (renormalize) {
#pragma unroll
    for (int s = 0; s < EPL; ++s) part += ex[s];
  } else {
#pragma unroll
    for (int s = 0; s < EPL; ++s)
      if (s * kWave + lane < E) part += expf(val[s] - top);
  }
  const float denom = wave_sum_f32(part);
#pragma unroll
  for (int s = 0; s < EPL; ++s) {
    const int j = s * kWave + lane;
    if (j < k) {
      ids[(int64_t)t * k + j] = seli[s];
      w[(int64_t)t * k + j] = ex[s] / denom;
    }
  }
}

hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, int bias_mode, int32_t* ids, float* w, hipStream_t s,
                        const float* part, int S, float* logits_out) {
  if (part && (S < 1 || S > kRouteMaxSplits || !logits_out)) return hipErrorInvalidValue;
  const int sel = bias != nullptr && bias_mode == 1;
  if (T <= 0) return hipSuccess;
  const int per_block = 4;  // tokens (wavefronts) per block
  dim3 grid(ceil_div(T, per_block)), block(per_block * kWave);
  const int epl = ceil_div(E, kWave);
  if (epl <= 1)
    route_kernel<1><<<grid, block, 0, s>>>(logits, bias, T, E, k, renormalize, sel, ids, w, part, S, logits_out);
  else if (epl <= 2)
    route_kernel<2><<<grid, block, 0, s>>>(logits, bias, T, E, k, renormalize, sel, ids, w, part, S, logits_out);
  else if (epl <= 4)
    route_kernel<4><<<grid, block, 0, s>>>(logits, bias, T, E, k, renormalize, sel, ids, w, part, S, logits_out);
  else if (epl <= 8)
    route_kernel<8><<<grid, block, 0, s>>>(logits, bias, T, E, k, renormalize, sel, ids, w, part, S, logits_out);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, bias, T, E, k, renormalize, sel, ids, w, part, S, logits_out);
  return hipGetLastError();
}

}  // namespace moe
