// Weighted combine and restore of token order.
//
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §2 (the layer
// output is the sum of the selected experts' outputs times their normalised
// routing weights) and §7 (expert outputs return to their tokens, are weighted
// by the router and put back in the original order).
//
// One block per token; each thread owns 16-byte chunks of the hidden vector and
// gathers the token's kept packed rows in slot order, accumulating in fp32 (the
// always-on expert's row, when present, is added last with weight 1).  The sum
// order is fixed, so results are deterministic.  HBM-bound: reads the kept rows
// once and writes y once.
#include "common.hpp"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yp,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w,
                                                      const void* __restrict__ ys,
                                                      const int32_t* __restrict__ ys_row0,
                                                      int T, int H, int k,
                                                      void* __restrict__ y) {
  const int t = blockIdx.x;
  if (t >= T) return;
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nvec = H / EPV;
  const int64_t shared_row = ys ? (int64_t)(ys_row0 ? *ys_row0 : 0) + t : -1;
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[EPV];
#pragma unroll
    for (int i = 0; i < EPV; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int r = pos[(int64_t)t * k + j];
      if (r < 0) continue;
      const float g = w[(int64_t)t * k + j];
      const uint4 q = ((const uint4*)yp)[(int64_t)r * nvec + v];
      if (BF16) {
        const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += g * bf16_bits_to_f32((uint16_t)(qq[i] & 0xffffu));
          acc[2 * i + 1] += g * bf16_bits_to_f32((uint16_t)(qq[i] >> 16));
        }
      } else {
        acc[0] += g * __uint_as_float(q.x);
        acc[1] += g * __uint_as_float(q.y);
        acc[2] += g * __uint_as_float(q.z);
        acc[3] += g * __uint_as_float(q.w);
      }
    }
    if (shared_row >= 0) {
      const uint4 q = ((const uint4*)ys)[shared_row * nvec + v];
      if (BF16) {
        const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += bf16_bits_to_f32((uint16_t)(qq[i] & 0xffffu));
          acc[2 * i + 1] += bf16_bits_to_f32((uint16_t)(qq[i] >> 16));
        }
      } else {
        acc[0] += __uint_as_float(q.x);
        acc[1] += __uint_as_float(q.y);
        acc[2] += __uint_as_float(q.z);
        acc[3] += __uint_as_float(q.w);
      }
    }
    uint4 o;
    if (BF16) {
      o.x = f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
      o.y = f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
      o.z = f32_to_bf16_bits(acc[4]) | ((uint32_t)f32_to_bf16_bits(acc[5]) << 16);
      o.w = f32_to_bf16_bits(acc[6]) | ((uint32_t)f32_to_bf16_bits(acc[7]) << 16);
    } else {
      o.x = __float_as_uint(acc[0]);
      o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2]);
      o.w = __float_as_uint(acc[3]);
    }
    ((uint4*)y)[(int64_t)t * nvec + v] = o;
  }
}

hipError_t launch_combine(const void* yp, const int32_t* pos, const float* w, const void* ys,
                          const int32_t* ys_row0, int T, int H, int k, int bf16, void* y,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (bf16)
    combine_kernel<true><<<T, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
  else
    combine_kernel<false><<<T, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
