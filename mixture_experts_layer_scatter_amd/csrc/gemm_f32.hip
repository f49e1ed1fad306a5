// Grouped fp32 GEMMs on vector FMA: the fp32 storage path of the gate,
// gate-up (SiLU*mul) and down projections.  Same contract and tile map as the
// bf16 MFMA path (gemm_bf16.hip), for layers stored in fp32.  CDNA4's fp32
// MFMA rate equals its fp32 vector-FMA rate, so this path stays on FMA with
// LDS tiling.
//
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §1, §2 and §8
// (expert FFN with a gate projection, one grouped GEMM per expert);
// "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地" §2.1 (gate).
#include "common.hpp"

namespace moe {

constexpr int kFB = 32;  // tile rows, tile columns and k-step

template <int EPI, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GroupedGemm p) {
  __shared__ float sa[kFB][kFB + 1];
  __shared__ float sb[kFB][kFB + 1];
  __shared__ float sb2[kFB][kFB + 1];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int NT = (p.N + kFB - 1) / kFB;
  const int tile = blockIdx.x;
  int total = p.tile_start ? p.tile_start[p.G] : (p.static_rows + kFB - 1) / kFB * NT;
  if (tile >= total) return;
  int g = 0, row_base = 0, rows = p.static_rows, li = tile;
  if (p.tile_start) {
    int lo = 0, hi = p.G;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_start[mid] <= tile) lo = mid;
      else hi = mid;
    }
    g = lo;
    li = tile - p.tile_start[g];
    row_base = p.offsets[g];
    rows = p.offsets[g + 1] - row_base;
  }
  const int mt = (rows + kFB - 1) / kFB;
  const int m0 = (li % mt) * kFB, n0 = (li / mt) * kFB;
  const bool extra = p.tile_start && g >= p.G_routed;
  const float* B = (const float*)(extra ? p.b_extra : p.b) + (extra ? 0 : (int64_t)g * p.b_stride);
  const float* B2 = nullptr;
  if (EPI == EPI_SWIGLU)
    B2 = (const float*)(extra ? p.b2_extra : p.b2) + (extra ? 0 : (int64_t)g * p.b_stride);
  const float* A = (const float*)p.a;
  const int K = p.K;

  float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float acc2[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  for (int k0 = 0; k0 < K; k0 += kFB) {
    for (int i = threadIdx.x; i < kFB * kFB; i += 256) {
      const int r = i / kFB, c = i % kFB;
      const int kk = k0 + c;
      float va = 0.f, vb = 0.f, vb2 = 0.f;
      if (m0 + r < rows && kk < K) {
        const int prow = row_base + m0 + r;
        const int64_t src = GATHER ? p.row_map[prow] : prow;
        va = A[src * K + kk];
      }
      if (n0 + r < p.N && kk < K) {
        vb = B[(int64_t)(n0 + r) * K + kk];
        if (EPI == EPI_SWIGLU) vb2 = B2[(int64_t)(n0 + r) * K + kk];
      }
      sa[r][c] = va;
      sb[r][c] = vb;
      if (EPI == EPI_SWIGLU) sb2[r][c] = vb2;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kFB; ++c) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] += sa[ty * 2 + i][c] * sb[tx * 2 + j][c];
          if (EPI == EPI_SWIGLU) acc2[i][j] += sa[ty * 2 + i][c] * sb2[tx * 2 + j][c];
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lr = m0 + ty * 2 + i;
    if (lr >= rows) continue;
    const int64_t orow = (int64_t)row_base + lr;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + tx * 2 + j;
      if (col >= p.N) continue;
      float v = acc[i][j];
      if (EPI == EPI_SWIGLU) v = v / (1.0f + expf(-v)) * acc2[i][j];
      ((float*)p.c)[orow * p.ldc + col] = v;
    }
  }
}

void gemm_f32_tiling(int N, int* bm, int* nt) {
  *bm = kFB;
  *nt = (N + kFB - 1) / kFB;
}

hipError_t launch_gemm_f32(GemmKind kind, const GroupedGemm& p, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const bool gather = p.row_map != nullptr;
  if (kind == GEMM_GATE_UP) {
    if (gather) gemm_f32_kernel<EPI_SWIGLU, true><<<max_tiles, 256, 0, s>>>(p);
    else gemm_f32_kernel<EPI_SWIGLU, false><<<max_tiles, 256, 0, s>>>(p);
  } else {
    if (gather) gemm_f32_kernel<EPI_F32, true><<<max_tiles, 256, 0, s>>>(p);
    else gemm_f32_kernel<EPI_F32, false><<<max_tiles, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
