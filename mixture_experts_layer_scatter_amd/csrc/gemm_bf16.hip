// Grouped bf16 GEMMs on CDNA4 MFMA: the router gate, the experts' gate-up
// projection with the SiLU*mul epilogue, and the experts' down projection.
//
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §8: after the
// count/sort/pack step, each expert runs one GEMM over the tokens it collected
// (a grouped GEMM); §1 and §2: each expert is an FFN from the hidden size to an
// inner size and back, with an added gate projection (SwiGLU: W2 (silu(W1 x) *
// W3 x)).  "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地"
// §2.1: the gate is a linear map from hidden size to experts without bias.
//
// Design for gfx950:
//  * C[r, n] = sum_k A[r, k] * B[n, k]; both operands are contiguous along k,
//    so one 16-byte load gives an MFMA lane its 8 consecutive k values.
//  * Block tile BM x BN, k-step 64, v_mfma_f32_32x32x16_bf16 with fp32
//    accumulators; WM x WN wavefronts, each owning a (BM/WM) x (BN/WN) tile.
//  * Operand tiles go HBM -> LDS with buffer_load ... lds (16 bytes per lane,
//    no VGPR staging), STAGES deep.  An LDS row holds 64 bf16 = eight 16-byte
//    chunks; chunk c of row r is stored at chunk c ^ (r & 7), so the eight
//    rows an MFMA fragment read touches fall in distinct banks.
//  * Buffer loads return zero past the resource's size and for the
//    out-of-range offset used for rows beyond a group: ragged row tails and
//    column tails need no branches.
//  * Groups (experts) have ragged row counts known only on the device.  A
//    device tile map (tile_start) lists every group's tiles; a persistent grid
//    walks it.  Tiles are dealt out XCD by XCD (workgroups go round-robin over
//    the 8 XCDs), so the workgroups sharing one XCD's L2 take consecutive tiles;
//    inside a group, tiles run column-group by column-group (GN column tiles x
//    all row tiles), so concurrent tiles reuse the same weight and row panels.
//  * Gate-up: the B tile interleaves 32-row blocks of W1 and W3, so each
//    wavefront holds W1 x and W3 x for the same columns in registers and
//    applies silu(a) * g before one bf16 store of the activation.
#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBK = 64;        // k elements per step
constexpr int kRowBytes = 128; // one LDS row of a k-step

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, 0, 0, 0);
}

// wait until at most n vector-memory operations of this wavefront are outstanding
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ float silu_f32(float a) { return a / (1.0f + __expf(-a)); }

constexpr uint32_t kOutOfRange = 0x80000000u;

template <int BM, int BN, int WM, int WN, int STAGES, int EPI, bool GATHER, int GN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int kWaves = WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_LOADS = BM / 8 / kWaves;  // 1 KB wave loads per stage
  static constexpr int B_LOADS = BN / 8 / kWaves;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is a multiple of 32x32");
  static_assert(A_LOADS * kWaves * 8 == BM && B_LOADS * kWaves * 8 == BN, "load split");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs W1/W3 column blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int n_max>
__device__ __forceinline__ void wait_outstanding(int n) {
  // n in [0, n_max]; unrolled to immediate waits
  if constexpr (n_max <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= n_max) wait_vmcnt<n_max>();
    else wait_outstanding<n_max - 1>(n);
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int EPI, bool GATHER, int GN>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_bf16_kernel(GroupedGemm p) {
  using C = GemmCfg<BM, BN, WM, WN, STAGES, EPI, GATHER, GN>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int wm = wid / WN, wn = wid % WN;
  const int K = p.K, KT = K / kBK;
  const int NT = (EPI == EPI_SWIGLU) ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;

  int total;
  if (p.tile_start) total = p.tile_start[p.G];
  else total = (p.static_rows + BM - 1) / BM * NT;
  const int nx = gridDim.x / 8, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = (total + 7) / 8;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a, (uint32_t)(p.a_rows * K * 2));

  for (int it = slot; it < per_xcd; it += nx) {
    const int tile = xcd * per_xcd + it;
    if (tile >= total) break;
    // ---- locate the tile: group, row tile, column tile -----------------------------------
    int g = 0, row_base = 0, rows = p.static_rows, li = tile;
    if (p.tile_start) {
      int lo = 0, hi = p.G;  // largest g with tile_start[g] <= tile
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
    const int mt = (rows + BM - 1) / BM;
    const int nblk = li / (mt * GN), rem = li % (mt * GN);
    const int m_t = rem % mt, n_t = nblk * GN + rem / mt;
    const int m0 = m_t * BM;
    const int rows_here = min(BM, rows - m0);

    const bool extra = p.tile_start && g >= p.G_routed;
    const char* bbase = (const char*)(extra ? p.b_extra : p.b) +
                        (extra ? 0 : (int64_t)g * p.b_stride * 2);
    const char* b2base = nullptr;
    if (EPI == EPI_SWIGLU)
      b2base = (const char*)(extra ? p.b2_extra : p.b2) + (extra ? 0 : (int64_t)g * p.b_stride * 2);
    const uint32_t b_bytes = (uint32_t)((int64_t)p.N * K * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(bbase, b_bytes);
    const __amdgpu_buffer_rsrc_t rB2 = make_rsrc(EPI == EPI_SWIGLU ? b2base : bbase, b_bytes);

    // ---- per-thread source offsets of the rows this thread loads -------------------------
    // wave load i covers tile rows (wid*A_LOADS + i)*8 + lane/8, chunk lane%8 (stored swizzled)
    const int chunk_phys = lane & 7;
    const int chunk_log = chunk_phys ^ ((lane >> 3) & 7);
    uint32_t a_off[C::A_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int r = (wid * C::A_LOADS + i) * 8 + (lane >> 3);
      uint32_t off = kOutOfRange;
      if (r < rows_here) {
        const int prow = row_base + m0 + r;
        const int64_t src = GATHER ? (int64_t)p.row_map[prow] : (int64_t)prow;
        off = (uint32_t)(src * K * 2) + chunk_log * 16;
      }
      a_off[i] = off;
    }
    uint32_t b_off[C::B_LOADS];
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int n = (wid * C::B_LOADS + i) * 8 + (lane >> 3);
      int src;
      if (EPI == EPI_SWIGLU) src = n_t * (BN / 2) + (n >> 6) * 32 + (n & 31);
      else src = n_t * BN + n;
      b_off[i] = src < p.N ? (uint32_t)src * (uint32_t)K * 2u + chunk_log * 16 : kOutOfRange;
    }

    auto issue = [&](int kt, int st) {
      char* sa = smem + st * C::STAGE_BYTES;
      char* sb = sa + C::A_BYTES;
      const uint32_t kb = (uint32_t)kt * kRowBytes;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i)
        load_lds16(rA, sa + (wid * C::A_LOADS + i) * 1024, a_off[i] + kb);
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) {
        const int blk = wid * C::B_LOADS + i;  // 8-row block; 4 of them per 32-row panel block
        if (EPI == EPI_SWIGLU && ((blk >> 2) & 1))
          load_lds16(rB2, sb + blk * 1024, b_off[i] + kb);
        else
          load_lds16(rB, sb + blk * 1024, b_off[i] + kb);
      }
    };

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    wait_vmcnt<0>();  // stores of the previous tile are out of the way
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < KT) issue(s, s);

    const int hi = lane >> 5, l32 = lane & 31;
    for (int kt = 0; kt < KT; ++kt) {
      const int ahead = min(KT - 1 - kt, STAGES - 2);  // stages allowed to stay in flight
      wait_outstanding<(STAGES - 2) * C::LOADS>(ahead * C::LOADS);
      __syncthreads();
      if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
      const char* sa = smem + (kt % STAGES) * C::STAGE_BYTES;
      const char* sb = sa + C::A_BYTES;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int phys = ((kk * 2 + hi) ^ (l32 & 7)) * 16;
        bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          af[i] = *(const bf16x8*)(sa + (wm * C::WTM + i * 32 + l32) * kRowBytes + phys);
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          bfr[j] = *(const bf16x8*)(sb + (wn * C::WTN + j * 32 + l32) * kRowBytes + phys);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();  // every wavefront is done reading the operand tiles

    // ---- epilogue ------------------------------------------------------------------------
    // 32x32 accumulator layout: lane holds column l32, rows 8*(r/4) + 4*hi + r%4.
    // Indices are rebuilt from an opaque copy of the lane id so the compiler does not hoist
    // dozens of loop-invariant row offsets out of the tile loop (they would spill).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int eh = ln >> 5, ec = ln & 31;
    const int64_t out_row0 = (int64_t)row_base + m0;
    if constexpr (EPI == EPI_F32) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * eh + (r & 3);
          if (lr >= rows_here) continue;
#pragma unroll
          for (int j = 0; j < C::TN; ++j) {
            const int col = n_t * BN + wn * C::WTN + j * 32 + ec;
            if (col < p.N) ((float*)p.c)[(out_row0 + lr) * p.ldc + col] = acc[i][j][r];
          }
        }
    } else {
      // bf16 tile staged in LDS (16-byte chunks swizzled by row), then 16-byte row stores
      constexpr int OUTC = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns of the tile
      constexpr int RS = OUTC * 2;                            // staging row bytes
      static_assert(BM * RS <= C::LDS_BYTES, "staging fits in the operand buffers");
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * eh + (r & 3);
          char* srow = smem + lr * RS;
          if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < C::TN; j += 2) {
              const int col = wn * (C::WTN / 2) + (j / 2) * 32 + ec;
              const float h = silu_f32(acc[i][j][r]) * acc[i][j + 1][r];
              *(uint16_t*)(srow + ((((col >> 3) ^ (lr & 7)) << 4) | ((col & 7) << 1))) =
                  f32_to_bf16_bits(h);
            }
          } else {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              const int col = wn * C::WTN + j * 32 + ec;
              *(uint16_t*)(srow + ((((col >> 3) ^ (lr & 7)) << 4) | ((col & 7) << 1))) =
                  f32_to_bf16_bits(acc[i][j][r]);
            }
          }
        }
      __syncthreads();
      constexpr int QPR = OUTC / 8;  // 16-byte chunks per row
      const int col_base = n_t * OUTC;
      for (int idx = tid; idx < BM * QPR; idx += C::kThreads) {
        const int row = idx / QPR, q = idx % QPR;
        const int col = col_base + q * 8;
        if (row < rows_here && col < p.N) {
          const uint4 v = *(const uint4*)(smem + row * RS + ((q ^ (row & 7)) << 4));
          *(uint4*)((uint16_t*)p.c + (out_row0 + row) * p.ldc + col) = v;
        }
      }
      __syncthreads();  // staging read before the next tile's loads land in LDS
    }
  }
}

// ---- configurations ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int STAGES, int EPI, bool GATHER, int GN>
static hipError_t run(const GroupedGemm& p, int max_tiles, int num_cus, hipStream_t s) {
  using C = GemmCfg<BM, BN, WM, WN, STAGES, EPI, GATHER, GN>;
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, STAGES, EPI, GATHER, GN>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  if (max_tiles <= 0) return hipSuccess;
  int per_cu = (160 * 1024) / C::LDS_BYTES;
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 2) per_cu = 2;
  int grid = num_cus * per_cu;
  if (grid > max_tiles) grid = max_tiles;
  grid = (grid + 7) / 8 * 8;
  kern<<<grid, C::kThreads, C::LDS_BYTES, s>>>(p);
  return hipGetLastError();
}

// choose tiles for a kind of GEMM from the rows a group holds on average
void gemm_bf16_tiling(GemmKind kind, int avg_rows_per_group, int N, int* bm, int* nt) {
  if (kind == GEMM_GATE) {
    const int bn = N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
    *bm = 32;
    *nt = (N + bn - 1) / bn;
    return;
  }
  const bool big = avg_rows_per_group >= 128;
  *bm = big ? 256 : 32;
  *nt = kind == GEMM_GATE_UP ? (N + 127) / 128 : (N + 255) / 256;
}

hipError_t launch_gemm_bf16(GemmKind kind, const GroupedGemm& p, int avg_rows_per_group,
                            int num_cus, hipStream_t s) {
  int bm, nt;
  gemm_bf16_tiling(kind, avg_rows_per_group, p.N, &bm, &nt);
  // upper bound of the tile count (the exact count is on the device)
  int64_t max_tiles;
  if (p.tile_start) {
    max_tiles = ((p.max_rows + bm - 1) / bm + p.G) * nt;
  } else {
    max_tiles = (int64_t)((p.static_rows + bm - 1) / bm) * nt;
  }
  if (max_tiles > (1 << 30)) max_tiles = 1 << 30;
  const int mt = (int)max_tiles;
  if (kind == GEMM_GATE) {
    if (p.N <= 32) return run<32, 32, 1, 1, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 64) return run<32, 64, 1, 2, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 128) return run<32, 128, 1, 4, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    return run<32, 256, 1, 4, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
  }
  const bool big = bm == 256;
  if (kind == GEMM_GATE_UP) {
    const bool gather = p.row_map != nullptr;
    if (big)
      return gather ? run<256, 256, 2, 2, 2, EPI_SWIGLU, true, 8>(p, mt, num_cus, s)
                    : run<256, 256, 2, 2, 2, EPI_SWIGLU, false, 8>(p, mt, num_cus, s);
    return gather ? run<32, 256, 1, 4, 4, EPI_SWIGLU, true, 1>(p, mt, num_cus, s)
                  : run<32, 256, 1, 4, 4, EPI_SWIGLU, false, 1>(p, mt, num_cus, s);
  }
  if (big) return run<256, 256, 2, 2, 2, EPI_BF16, false, 8>(p, mt, num_cus, s);
  return run<32, 256, 1, 4, 4, EPI_BF16, false, 1>(p, mt, num_cus, s);
}

}  // namespace moe
