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
// once and writes y once.  With few tokens (decode) a token's vector is split over
// several blocks, one chunk per thread, and each thread reads the slot indices and
// weights eight at a time and issues their rows' loads before adding any of them: a
// block per token would leave every thread a chain of dependent loads (one per
// slot and chunk) with too few blocks to overlap them.  Both kernels add the same
// terms in the same order, so they agree bit for bit.
#include "common.hpp"

namespace moe {

template <bool BF16, int EPV>
__device__ __forceinline__ void add_chunk(float (&acc)[EPV], uint4 q, float g) {
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

// tokens below this count take the split kernel
constexpr int kCombineSplitBelow = 2048;

// grid (T, ceil(nvec / 256)): thread (blockIdx.y * 256 + threadIdx.x) owns one chunk of token
// blockIdx.x; the same terms in the same order as combine_kernel
template <bool BF16>
__global__ __launch_bounds__(256) void combine_split_kernel(const void* __restrict__ yp,
                                                            const int32_t* __restrict__ pos,
                                                            const float* __restrict__ w,
                                                            const void* __restrict__ ys,
                                                            const int32_t* __restrict__ ys_row0,
                                                            int T, int H, int k,
                                                            void* __restrict__ y) {
  const int t = blockIdx.x;
  constexpr int EPV = BF16 ? 8 : 4;
  const int nvec = H / EPV;
  const int v = blockIdx.y * blockDim.x + threadIdx.x;
  if (t >= T || v >= nvec) return;
  float acc[EPV];
#pragma unroll
  for (int i = 0; i < EPV; ++i) acc[i] = 0.f;
  const uint4* rows = (const uint4*)yp;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int r[8];
    float g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r[u] = j0 + u < k ? pos[(int64_t)t * k + j0 + u] : -1;
      g[u] = j0 + u < k ? w[(int64_t)t * k + j0 + u] : 0.f;
    }
    uint4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      q[u] = r[u] >= 0 ? rows[(int64_t)r[u] * nvec + v] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r[u] >= 0) add_chunk<BF16, EPV>(acc, q[u], g[u]);
  }
  if (ys) {
    const int64_t srow = (int64_t)(ys_row0 ? *ys_row0 : 0) + t;
    const uint4 q = ((const uint4*)ys)[srow * nvec + v];
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

hipError_t launch_combine(const void* yp, const int32_t* pos, const float* w, const void* ys,
                          const int32_t* ys_row0, int T, int H, int k, int bf16, void* y,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T < kCombineSplitBelow) {
    const int nvec = H / (bf16 ? 8 : 4);
    const dim3 grid(T, (nvec + 255) / 256);
    if (bf16)
      combine_split_kernel<true><<<grid, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
    else
      combine_split_kernel<false><<<grid, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
    return hipGetLastError();
  }
  if (bf16)
    combine_kernel<true><<<T, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
  else
    combine_kernel<false><<<T, 256, 0, s>>>(yp, pos, w, ys, ys_row0, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
