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
// Design for gfx950 (two kernels share the conventions below):
//  * C[r, n] = sum_k A[r, k] * B[n, k]; both operands are contiguous along k,
//    so one 16-byte load gives an MFMA lane its 8 consecutive k values.
//  * v_mfma_f32_32x32x16_bf16 with fp32 accumulators, k-step 64.
//  * Operand tiles go HBM -> LDS with buffer_load ... lds (16 bytes per lane,
//    no VGPR staging).  An LDS row holds 64 bf16 = eight 16-byte chunks; chunk
//    c of row r is stored at chunk c ^ swz(r), so the rows one MFMA fragment
//    read touches fall in distinct banks.
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
//
// Prefill kernel (gemm_big_kernel, rows per group >= 128): 256 x 256 tiles,
// 8 wavefronts (two per SIMD, each 128 token rows x 64 columns), two LDS
// stages.  The weights are the MFMA's first operand, so each lane ends with 4
// consecutive output columns of one token row and stores them straight from
// registers; the next tile's first loads go out before that epilogue.  The
// barrier inside the k-loop leaves the loads of the stage in flight alone
// (s_barrier without a memory-counter drain).  Rows past a group's end load as
// zeros, so every tile costs the same and the workgroups of an XCD stay in
// step over the panels they share.
//
// Small-group kernel (gemm_bf16_kernel, decode and the gate): 32-row tiles,
// four wavefronts across the columns, four LDS stages to keep weight bytes in
// flight; the activation tile is staged through LDS for 16-byte row stores.
#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBK = 64;        // k elements per step
constexpr int kRowBytes = 128; // one LDS row of a k-step

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                           int soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// wait until at most n vector-memory operations of this wavefront are outstanding
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8,
// vmcnt[5:4] bits 15:14); "no wait" is the field's maximum
template <int n>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(n >= 0 && n < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xf | (0x3 << 14) | (0x7 << 4) | (n << 8));
}

// Workgroup barrier that leaves outstanding global->LDS loads in flight (the caller has waited
// for exactly what it needs); also a compiler fence, so no LDS access moves across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// silu(a) = a * sigmoid(a) with the hardware exp2 and reciprocal (the result is rounded to bf16)
__device__ __forceinline__ float silu_fast(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// swizzle of the 16-byte chunks of a 128-byte LDS row: distinct banks for the 8 (and the 16)
// consecutive rows that one fragment read serves per cycle
__device__ __forceinline__ int row_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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

  int total_base;
  if (p.tile_start) total_base = p.tile_start[p.G];
  else total_base = (p.static_rows + BM - 1) / BM * NT;
  // split-K: ksplit consecutive copies of the tile list, copy ks reducing over its share of
  // the k-steps into the partial output c + ks * c_split_stride
  const int ks_n = p.ksplit > 1 ? p.ksplit : 1;
  const int total = total_base * ks_n;
  const int nx = gridDim.x / 8, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per_xcd = (total + 7) / 8;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a, (uint32_t)(p.a_rows * K * 2));

  for (int it = slot; it < per_xcd; it += nx) {
    const int tile_all = xcd * per_xcd + it;
    if (tile_all >= total) break;
    const int ks = tile_all / total_base, tile = tile_all - ks * total_base;
    const int kt0 = (int)((int64_t)ks * KT / ks_n), kt1 = (int)((int64_t)(ks + 1) * KT / ks_n);
    const int KTL = kt1 - kt0;  // k-steps of this tile
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

    auto issue = [&](int lk, int st) {
      char* sa = smem + st * C::STAGE_BYTES;
      char* sb = sa + C::A_BYTES;
      const uint32_t kb = (uint32_t)(kt0 + lk) * kRowBytes;
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
      if (s < KTL) issue(s, s);

    const int hi = lane >> 5, l32 = lane & 31;
    for (int kt = 0; kt < KTL; ++kt) {
      const int ahead = min(KTL - 1 - kt, STAGES - 2);  // stages allowed to stay in flight
      wait_outstanding<(STAGES - 2) * C::LOADS>(ahead * C::LOADS);
      wait_lgkmcnt<0>();
      barrier_keep_loads();  // later stages stay in flight
      if (kt + STAGES - 1 < KTL) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
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
            if (col < p.N)
              ((float*)p.c + ks * p.c_split_stride)[(out_row0 + lr) * p.ldc + col] = acc[i][j][r];
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

// ---- prefill kernel ----------------------------------------------------------------------------

namespace big {
constexpr int BM = 256, BN = 256, WM = 2, WN = 4, WAVES = WM * WN, THREADS = WAVES * kWave;
constexpr int WTN = BN / WN;            // 64 columns per wavefront
constexpr int TM = BM / WM / 32;        // 4 token blocks of 32 rows per wavefront
constexpr int TN = WTN / 32;            // 2 column blocks of 32
constexpr int KK = kBK / 16;            // MFMA k-steps per LDS stage
constexpr int RPL = 1024 / kRowBytes;   // rows one 1 KB wavefront load covers
constexpr int A_LOADS = BM / RPL / WAVES, B_LOADS = BN / RPL / WAVES, L = A_LOADS + B_LOADS;
constexpr int A_BYTES = BM * kRowBytes, STAGE = (BM + BN) * kRowBytes;
constexpr int LDS = 2 * STAGE;          // two stages: 128 KB
static_assert(A_LOADS * RPL * WAVES == BM && B_LOADS * RPL * WAVES == BN, "load split");
static_assert(LDS <= 160 * 1024, "LDS budget");
}  // namespace big

template <int EPI, bool GATHER, int GN>
__global__ __launch_bounds__(big::THREADS) void gemm_big_kernel(GroupedGemm p) {
  using namespace big;
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_BF16, "bf16 outputs only");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid / WN, wn = wid % WN;
  const int K = p.K, KT = K / kBK;
  const int total = p.tile_start[p.G];
  const int nx = gridDim.x / 8, xcd = blockIdx.x % 8;
  const int per_xcd = (total + 7) / 8;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a, (uint32_t)(p.a_rows * K * 2));

  const int l32 = lane & 31, hi = lane >> 5;
  const int sw = row_swizzle(l32);
  const uint32_t a_frag = (uint32_t)((wm * (BM / WM) + l32) * kRowBytes);
  const uint32_t b_frag = (uint32_t)(A_BYTES + (wn * WTN + l32) * kRowBytes);

  struct Tile {
    int row_base, m0, rows_here, n_t, g;
  };
  auto locate = [&](int it, Tile& t) -> bool {
    if (it >= per_xcd) return false;
    const int tile = xcd * per_xcd + it;
    if (tile >= total) return false;
    int lo = 0, hi2 = p.G;  // largest g with tile_start[g] <= tile
    while (hi2 - lo > 1) {
      const int mid = (lo + hi2) >> 1;
      if (p.tile_start[mid] <= tile) lo = mid;
      else hi2 = mid;
    }
    const int g = lo, li = tile - p.tile_start[g];
    const int row_base = p.offsets[g], rows = p.offsets[g + 1] - row_base;
    const int mt = (rows + BM - 1) / BM;
    const int nblk = li / (mt * GN), rem = li % (mt * GN);
    t.g = g;
    t.row_base = row_base;
    t.m0 = (rem % mt) * BM;
    t.n_t = nblk * GN + rem / mt;
    t.rows_here = min(BM, rows - t.m0);
    return true;
  };

  // per-lane source offsets of the current tile's loads (lane: row lane / 8, chunk lane % 8)
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
  __amdgpu_buffer_rsrc_t rB, rB2;
  auto setup = [&](const Tile& t) {
    const bool extra = t.g >= p.G_routed;
    const char* bbase =
        (const char*)(extra ? p.b_extra : p.b) + (extra ? 0 : (int64_t)t.g * p.b_stride * 2);
    const char* b2base = bbase;
    if (EPI == EPI_SWIGLU)
      b2base = (const char*)(extra ? p.b2_extra : p.b2) + (extra ? 0 : (int64_t)t.g * p.b_stride * 2);
    const uint32_t b_bytes = (uint32_t)((int64_t)p.N * K * 2);
    rB = make_rsrc(bbase, b_bytes);
    rB2 = make_rsrc(b2base, b_bytes);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = (wid * A_LOADS + i) * RPL + lane / 8;
      const int c = (lane & 7) ^ row_swizzle(r);
      uint32_t off = kOutOfRange;
      if (r < t.rows_here) {
        const int prow = t.row_base + t.m0 + r;
        const int64_t src = GATHER ? (int64_t)p.row_map[prow] : (int64_t)prow;
        off = (uint32_t)(src * K * 2) + c * 16;
      }
      a_off[i] = off;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int n = (wid * B_LOADS + i) * RPL + lane / 8;
      const int c = (lane & 7) ^ row_swizzle(n);
      const int src = EPI == EPI_SWIGLU ? t.n_t * (BN / 2) + (n >> 6) * 32 + (n & 31) : t.n_t * BN + n;
      b_off[i] = src < p.N ? (uint32_t)src * (uint32_t)K * 2u + c * 16 : kOutOfRange;
    }
  };
  // stage kt into LDS slot `slot`; past the last stage every lane gets the out-of-range offset
  // (no memory access, zeros into a free slot), so every step issues the same number of loads
  auto issue = [&](int kt, int slot, bool valid) {
    char* sa = smem + slot * STAGE;
    char* sb = sa + A_BYTES;
    const int kb = valid ? kt * kRowBytes : 0;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      load_lds16(rA, sa + (wid * A_LOADS + i) * 1024, valid ? a_off[i] : kOutOfRange, kb);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int blk = wid * B_LOADS + i;
      const bool second = EPI == EPI_SWIGLU && (((blk * RPL) >> 5) & 1);
      load_lds16(second ? rB2 : rB, sb + blk * 1024, valid ? b_off[i] : kOutOfRange, kb);
    }
  };

  f32x16 acc[TM][TN];
  bf16x8 fa[2][TM], fb[2][TN];

  // The k-loop.  At the barrier in the middle of step kt every wavefront has read all of
  // stage kt, whose slot then takes stage kt + 2 while the last MFMAs of step kt run from
  // registers.  Every tile costs the same (rows past a group's end are zeros), which keeps the
  // workgroups of an XCD in step, so the operand panels they share are fetched into L2 once.
  auto read_frags = [&](const char* st, int kk, int buf) {
    const uint32_t coff = (uint32_t)(((kk * 2 + hi) ^ sw) * 16);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = *(const bf16x8*)(st + a_frag + coff + i * 32 * kRowBytes);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = *(const bf16x8*)(st + b_frag + coff + j * 32 * kRowBytes);
  };
  // weights as the first operand: D[column][token]
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
  };
  auto kloop = [&]() {
    read_frags(smem, 0, 0);
    if (1 < KT) issue(1, 1, true);
    for (int kt = 0; kt < KT; ++kt) {
      const char* cur = smem + (kt & 1) * STAGE;
      const char* nxt = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk < KK - 1) {
          read_frags(cur, kk + 1, (kk + 1) & 1);
        } else {
          wait_vmcnt<0>();       // stage kt + 1 landed (this wavefront's share)
          wait_lgkmcnt<0>();     // this wavefront's reads of stage kt returned
          barrier_keep_loads();  // ... and everyone else's
          read_frags(nxt, 0, 0);
          issue(kt + 2, kt & 1, kt + 2 < KT);
        }
        mfmas(kk & 1);
        // interleave: one MFMA, then one LDS read and (after the barrier) one global load
#pragma unroll
        for (int m = 0; m < TM * TN; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (m < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (kk == KK - 1 && m < L) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
    }
  };

  int it = blockIdx.x / 8;
  Tile cur;
  if (!locate(it, cur)) return;
  setup(cur);
  issue(0, 0, true);

  while (true) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    wait_vmcnt<0>();  // stage 0 (and the previous tile's stores)
    barrier_keep_loads();
    kloop();
    // everyone is done with the operand slots and the loads past the last stage have landed
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_keep_loads();

    const Tile done = cur;
    it += nx;
    const bool more = locate(it, cur);
    if (more) {  // the next tile's first stage loads while this tile's results go out
      setup(cur);
      issue(0, 0, true);
    }

    // epilogue: lane holds token l32 of block i and columns 8q + 4hi + (0..3) of each
    // 32-column block j
    const int64_t out_row0 = (int64_t)done.row_base + done.m0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int tok = wm * (BM / WM) + i * 32 + l32;
      if (tok >= done.rows_here) continue;
      uint16_t* crow = (uint16_t*)p.c + (out_row0 + tok) * p.ldc;
      if constexpr (EPI == EPI_SWIGLU) {
        // blocks j (W1) and j + 1 (W3) hold the same 32 columns
#pragma unroll
        for (int j = 0; j < TN; j += 2)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = done.n_t * (BN / 2) + wn * (WTN / 2) + (j / 2) * 32 + 8 * q + 4 * hi;
            if (col < p.N) {
              float h[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) h[e] = silu_fast(acc[i][j][4 * q + e]) * acc[i][j + 1][4 * q + e];
              uint2 v;
              v.x = pack_bf16x2(h[0], h[1]);
              v.y = pack_bf16x2(h[2], h[3]);
              *(uint2*)(crow + col) = v;
            }
          }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = done.n_t * BN + wn * WTN + j * 32 + 8 * q + 4 * hi;
            if (col < p.N) {
              uint2 v;
              v.x = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
              v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              *(uint2*)(crow + col) = v;
            }
          }
      }
    }
    if (!more) break;
  }
}

template <int EPI, bool GATHER>
static hipError_t run_big(const GroupedGemm& p, int max_tiles, int num_cus, hipStream_t s) {
  auto kern = gemm_big_kernel<EPI, GATHER, 8>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, big::LDS);
  if (e != hipSuccess) return e;
  if (max_tiles <= 0) return hipSuccess;
  int grid = num_cus;  // one workgroup (8 wavefronts, 128 KB of LDS) per CU
  if (grid > max_tiles) grid = max_tiles;
  grid = (grid + 7) / 8 * 8;
  kern<<<grid, big::THREADS, big::LDS, s>>>(p);
  return hipGetLastError();
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
  if (p.ksplit > 1) max_tiles *= p.ksplit;
  if (max_tiles > (1 << 30)) max_tiles = 1 << 30;
  const int mt = (int)max_tiles;
  if (kind == GEMM_GATE) {
    if (p.N <= 32) return run<32, 32, 1, 1, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 64) return run<32, 64, 1, 2, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 128) return run<32, 128, 1, 4, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
    return run<32, 256, 1, 4, 4, EPI_F32, false, 1>(p, mt, num_cus, s);
  }
  const bool big = bm == 256;
  if (big && !p.tile_start) return hipErrorInvalidValue;  // the prefill kernel walks a tile map
  if (kind == GEMM_GATE_UP) {
    const bool gather = p.row_map != nullptr;
    if (big)
      return gather ? run_big<EPI_SWIGLU, true>(p, mt, num_cus, s)
                    : run_big<EPI_SWIGLU, false>(p, mt, num_cus, s);
    return gather ? run<32, 256, 1, 4, 4, EPI_SWIGLU, true, 1>(p, mt, num_cus, s)
                  : run<32, 256, 1, 4, 4, EPI_SWIGLU, false, 1>(p, mt, num_cus, s);
  }
  if (big) return run_big<EPI_BF16, false>(p, mt, num_cus, s);
  return run<32, 256, 1, 4, 4, EPI_BF16, false, 1>(p, mt, num_cus, s);
}

// ---- split-K reduction: out[i] = sum over s = 0..S-1 of part[s * n + i], in that order ----------
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                           int64_t n, float* __restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float acc = part[i];
    for (int s = 1; s < S; ++s) acc += part[s * n + i];
    out[i] = acc;
  }
}

hipError_t launch_splitk_reduce(const float* part, int S, int64_t n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  splitk_reduce_kernel<<<(int)blocks, 256, 0, s>>>(part, S, n, out);
  return hipGetLastError();
}

}  // namespace moe
