// Per-row FP8 E4M3 quantisation of expert weights.
//
// "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地" §5.2 serves
// the experts with 8-bit-class weights (its configuration names 4-bit weights
// with FP8 activations) to cut the weight bytes a decode step streams.  Here:
// E4M3 codes (the OCP format gfx950's conversions implement: bias 7, largest
// finite 448, no infinities) with one fp32 scale per row of a linear layer's
// [out, in] weight:
//   scale[r] = amax_k |w[r,k]| / 448   (one correctly rounded fp32 division)
//   q[r,k]   = E4M3 nearest to w[r,k] / scale[r], ties to even, saturating.
// The rounding is the hardware conversion's (round to nearest even); the
// quotient is clamped to +-448 first, so a quotient a rounding step above 448
// saturates instead of becoming NaN.
//
// One 256-thread block per row (grid-stride over rows); 8 elements per thread
// step, 8-byte code stores.
#include "common.hpp"

namespace moe {

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* __restrict__ w,
                                                           int64_t rows, int K,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales) {
  __shared__ float red[256 / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    auto load8 = [&](int k, float (&v)[8]) {
      if constexpr (BF16) {
        const uint4 u = *(const uint4*)((const uint16_t*)w + r * K + k);
        const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = __uint_as_float(h[i] << 16);
          v[2 * i + 1] = __uint_as_float(h[i] & 0xffff0000u);
        }
      } else {
        const float4 a = *(const float4*)((const float*)w + r * K + k);
        const float4 b = *(const float4*)((const float*)w + r * K + k + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    };
    // row maximum of |w| (max is exact in any order)
    float m = 0.f;
    for (int k = tid * 8; k < K; k += 256 * 8) {
      float v[8];
      load8(k, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if (lane == 0) red[wid] = m;
    __syncthreads();
    float amax = red[0];
#pragma unroll
    for (int i = 1; i < 256 / kWave; ++i) amax = fmaxf(amax, red[i]);
    __syncthreads();  // red is rewritten for the next row
    const float scale = amax / 448.0f;
    if (tid == 0) scales[r] = scale;
    for (int k = tid * 8; k < K; k += 256 * 8) {
      float v[8];
      load8(k, v);
      uint32_t packed[2] = {0u, 0u};
      if (scale != 0.f) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = fminf(fmaxf(v[4 * h + i] / scale, -448.f), 448.f);
          int p = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          p = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], p, true);
          packed[h] = (uint32_t)p;
        }
      }
      *(uint2*)(q + r * K + k) = make_uint2(packed[0], packed[1]);
    }
  }
}

hipError_t launch_quantize_fp8(const void* w, int bf16, int64_t rows, int K, uint8_t* q,
                               float* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int grid = rows < 65536 ? (int)rows : 65536;
  if (bf16)
    quantize_fp8_kernel<true><<<grid, 256, 0, s>>>(w, rows, K, q, scales);
  else
    quantize_fp8_kernel<false><<<grid, 256, 0, s>>>(w, rows, K, q, scales);
  return hipGetLastError();
}

}  // namespace moe
