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

// MXFP4 (the OCP microscaling format's E2M1 elements, one E8M0 scale per 32 consecutive k):
// per block, shared = clamp(floor(log2(amax)) - 2, -126, 127) (2 = the largest E2M1 exponent),
// scale code shared + 127 (127 for a zero block), and each element the E2M1 code nearest to
// w / 2^shared, ties to even, saturating at +-6 (the hardware's scaled conversion, which
// divides by the scale).  One thread per block of 32; codes two per byte, low nibble first.
// Both arrays are stored blocked by 32 rows and 128 k, the piece of a weight tile one stage of
// the grouped GEMM reads: the 64 code bytes of a row's 128-k span follow those of the previous
// row, so a 32-row block's span is 2 KB of whole lines; the four scales of a row's span sit in
// one dword, and the dwords of 32 rows fill one 128-byte line.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const void* __restrict__ w,
                                                             int64_t blocks, int K,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scales) {
  const int nb = K / 32, spans = K / 128;
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < blocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    float v[32];
    if constexpr (BF16) {
      const uint4* src = (const uint4*)((const uint16_t*)w + b * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = src[i];
        const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = __uint_as_float(h[j] << 16);
          v[8 * i + 2 * j + 1] = __uint_as_float(h[j] & 0xffff0000u);
        }
      }
    } else {
      const float4* src = (const float4*)((const float*)w + b * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    uint8_t code = 127;
    if (amax > 0.f) {
      // amax = m * 2^e with m in [0.5, 1): floor(log2(amax)) = e - 1
      int shared = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;
      shared = shared < -126 ? -126 : (shared > 127 ? 127 : shared);
      code = (uint8_t)(shared + 127);
      const float scale = __uint_as_float((uint32_t)code << 23);  // 2^shared, a normal float
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t r = 0;
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 0], v[8 * d + 1], scale, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 2], v[8 * d + 3], scale, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 4], v[8 * d + 5], scale, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 6], v[8 * d + 7], scale, 3);
        packed[d] = r;
      }
    }
    const int64_t row = b / nb;
    const int kb = (int)(b - row * nb);
    const int64_t span = (row >> 5) * spans + (kb >> 2);
    *(uint4*)(q + span * 2048 + (row & 31) * 64 + (kb & 3) * 16) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
    scales[span * 128 + (row & 31) * 4 + (kb & 3)] = code;
  }
}

hipError_t launch_quantize_mxfp4(const void* w, int bf16, int64_t rows, int K, uint8_t* q,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (K / 32);
  if (blocks <= 0) return hipSuccess;
  const int64_t g = (blocks + 255) / 256;
  const int grid = g < 65536 ? (int)g : 65536;
  if (bf16)
    quantize_mxfp4_kernel<true><<<grid, 256, 0, s>>>(w, blocks, K, q, scales);
  else
    quantize_mxfp4_kernel<false><<<grid, 256, 0, s>>>(w, blocks, K, q, scales);
  return hipGetLastError();
}

// MXFP8 activations: one thread per block of 32 consecutive elements of a row; the codes stay
// row-major (32 bytes per block, two 16-byte stores) and so do the scales (one byte per block).
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const void* __restrict__ x,
                                                             int64_t blocks,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ scales) {
  for (int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; b < blocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    float v[32];
    if constexpr (BF16) {
      const uint4* src = (const uint4*)((const uint16_t*)x + b * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = src[i];
        const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = __uint_as_float(h[j] << 16);
          v[8 * i + 2 * j + 1] = __uint_as_float(h[j] & 0xffff0000u);
        }
      }
    } else {
      const float4* src = (const float4*)((const float*)x + b * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t code = mxfp8_scale_code(amax);
    uint32_t w[8];
#pragma unroll
    for (int d = 0; d < 8; ++d)
      w[d] = amax > 0.f ? mxfp8_pack4(v[4 * d], v[4 * d + 1], v[4 * d + 2], v[4 * d + 3], code) : 0u;
    uint4* dst = (uint4*)(q + b * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[b] = (uint8_t)code;
  }
}

hipError_t launch_quantize_mxfp8(const void* x, int bf16, int64_t rows, int K, uint8_t* q,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (K / 32);
  if (blocks <= 0) return hipSuccess;
  const int64_t g = (blocks + 255) / 256;
  const int grid = g < 65536 ? (int)g : 65536;
  if (bf16)
    quantize_mxfp8_kernel<true><<<grid, 256, 0, s>>>(x, blocks, q, scales);
  else
    quantize_mxfp8_kernel<false><<<grid, 256, 0, s>>>(x, blocks, q, scales);
  return hipGetLastError();
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
