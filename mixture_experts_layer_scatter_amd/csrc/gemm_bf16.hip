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
// One kernel template serves all three (gemm_kernel), in these shapes:
//  * prefill (a group holds >= 128 rows on average): 256 x 256 tiles, 8
//    wavefronts (two per SIMD, each 128 token rows x 64 columns), two LDS
//    slots for the token-row tile and three for the weight tile (160 KB);
//  * decode and the gate: 32-row tiles, up to 4 wavefronts across the columns,
//    four LDS stages to keep weight bytes in flight;
//  * a split gate over many tokens: 128-row tiles, 4 wavefronts of 64 rows.
//
// Design for gfx950:
//  * C[r, n] = sum_k A[r, k] * B[n, k]; both operands are contiguous along k,
//    so one 16-byte load gives an MFMA lane its 8 consecutive k values.
//  * v_mfma_f32_32x32x16_bf16 with fp32 accumulators, k-step 64.  The weights
//    are the MFMA's first operand (D[column][token]), so each lane ends with 4
//    consecutive output columns of one token row and stores them straight from
//    registers (8 bytes bf16, 16 bytes fp32): no LDS staging, and the next
//    tile's first loads go out before the epilogue.
//  * Operand tiles go HBM -> LDS with buffer_load ... lds (16 bytes per lane,
//    no VGPR staging).  An LDS row holds 64 bf16 = eight 16-byte chunks; chunk
//    c of row r is stored at chunk c ^ swz(r), so the rows one fragment read
//    serves per cycle fall in distinct banks.
//  * At the barrier in the middle of step kt every wavefront has read all of
//    stage kt, whose slots then take the token rows of step kt + S and the
//    weights of step kt + SB right away; the barrier is a bare s_barrier that
//    leaves the stages in flight alone (a full __syncthreads would drain them).
//    Loads past the last stage carry the out-of-range offset (no memory access,
//    zeros into a free slot), so every step issues the same number of loads and
//    the wait count is a constant.
//  * Buffer loads return zero past the resource's size and for the
//    out-of-range offset used for rows beyond a group: ragged row tails and
//    column tails need no branches.  A group's 32-row blocks are spread evenly
//    over its row tiles and a wavefront skips the MFMAs of blocks without rows,
//    so the tiles of a group cost about the same, which keeps the workgroups of
//    an XCD in step over the operand panels they share.
//  * Groups (experts) have ragged row counts known only on the device.  A
//    device tile map (tile_start, with one entry per tile naming its group)
//    lists every group's tiles; a persistent grid walks it.  Tiles are dealt
//    out XCD by XCD (workgroups go round-robin over the 8 XCDs), so the
//    workgroups sharing one XCD's L2 take consecutive tiles;
//    inside a group, tiles run column-group by column-group (GN column tiles x
//    all row tiles), so concurrent tiles reuse the same weight and row panels.
//  * Gate-up: the B tile interleaves 32-row blocks of W1 and W3, so each
//    wavefront holds W1 x and W3 x for the same columns in registers and
//    applies silu(a) * g before one bf16 store of the activation.
//  * The gate (fp32 logits) can split its reduction over ksplit workgroups per
//    tile; the partial sums are added in a fixed order afterwards.
//  * MXFP4 weights (WQ = 2): E2M1 codes, two per byte, with an E8M0 scale per
//    32 k of a row, both stored blocked by 32 rows and 128 k (one stage of a
//    32-row block reads 2 KB of codes and one line of scales, all whole
//    lines); the code and scale tiles travel into LDS, and
//    a fragment read widens 8 codes with the hardware's scaled conversion (the
//    products are exact in bf16), so the scales never reach the epilogue.
//  * MXFP4 weights on MXFP8 token rows (WQ = 3, "MoE 推理架构深度实战" §5.2's 4-bit weights
//    with FP8 activations): both operands stay in their codes and the block-scaled MFMA
//    (v_mfma_scale_f32_32x32x64_f8f6f4) applies each lane's E8M0 scales; the gate-up epilogue
//    quantises silu(a) * g to MXFP8 for the down GEMM (EPI_SWIGLU_MX8).
//  * FP8 weights (WQ = 1): the weight tile travels HBM -> LDS as E4M3 bytes (half
//    the bytes of bf16, the point for the weight-streaming decode shape); a
//    fragment read takes 8 codes and widens them to bf16 in registers (every
//    E4M3 value is exact in bf16), so the same bf16 MFMA runs; the per-row scale
//    multiplies the fp32 accumulator in the epilogue (it factors out of the sum).
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// one 16-byte-per-lane global->LDS load: the wavefront's 1 KB lands contiguously at `lds`
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
// the same with 4 bytes per lane (256 bytes per wavefront)
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                                          int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8,
// vmcnt[5:4] bits 15:14); a field at its maximum does not wait
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}
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

// Two quads of bf16 outputs of a token row, as the MFMA leaves them: lane half hi holds
// columns 4hi .. 4hi + 3 of quad a (dwords a0, a1) and of quad b, 8 columns further (b0, b1).
// One v_permlane32_swap per dword pair trades lane half 0's quad b for half 1's quad a, so
// lane half 0 ends with columns 0 .. 7 and half 1 with columns 8 .. 15: one 16-byte store per
// lane at column 8hi, in place of two 8-byte stores.
__device__ __forceinline__ uint4 swap_halves(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1) {
  // lanes 0..31 keep a and take lanes 32..63's a; lanes 32..63 keep b and take lanes 0..31's b
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return make_uint4(s0[0], s1[0], s0[1], s1[1]);
}

// Swizzle of the 16-byte chunks of an LDS row of CH chunks (chunk c of row r sits at c ^
// swizzle(r)): the 8 (and the 16) consecutive rows that one fragment read serves per cycle fall
// in distinct banks.  It depends on bits 0..4 of the row only, so the rows of a fragment's
// 32-row blocks share it.
template <int CH>
__device__ __forceinline__ int row_swizzle(int r) {
  static_assert(CH == 4 || CH == 8 || CH == 16, "rows of 64, 128 or 256 bytes");
  if constexpr (CH == 16) return r & 15;
  else if constexpr (CH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// eight E4M3 codes -> eight bf16 values (exact: the upper half of each fp32 conversion)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 v) {
  union {
    uint32_t u[4];
    bf16x8 h;
  } r;
  const uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);  // codes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);   // codes 2, 3
    r.u[2 * i] = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u);
    r.u[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u);
  }
  return r.h;
}

// eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times a power-of-two
// scale -> eight bf16 values (exact: E2M1 values have two significant bits)
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float scale) {
  union {
    uint32_t u[4];
    bf16x8 h;
  } r;
  r.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r.h;
}

template <int BM_, int BN_, int WM_, int WN_, int S_, int BK_ = 64, int SB_ = S_, int AE_ = 2>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
  static constexpr int AE = AE_;  // bytes of an A (token-row) element: 2 (bf16), 1 (MXFP8)
  // LDS stages of the weight operand (S: of the token rows).  With 256 x 256 tiles two full
  // stages take 128 KB of the 160 KB, so one operand can get a third slot: a step more of
  // latency for its L2 misses
  static constexpr int SB = SB_;
  static_assert(SB == S || (S == 2 && SB == 3) || (S == 3 && SB == 2), "stage counts");
  static constexpr int BK = BK_;                      // k elements per LDS stage
  static constexpr int ROWB = BK * AE, CH = ROWB / 16; // bytes and 16-byte chunks of an A row
  static constexpr int WAVES = WM * WN, THREADS = WAVES * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wavefront tile
  static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32 x 32 MFMA blocks per wavefront
  static constexpr int KK = BK / 16;                  // MFMA k-steps per LDS stage
  static constexpr int RPL = 1024 / ROWB;             // A rows one 1 KB wavefront load covers
  static constexpr int A_LOADS = BM / RPL / WAVES;
  static constexpr int A_BYTES = BM * ROWB;
  static_assert(BK == 64 || BK == 128, "k-step");
  static_assert(AE == 2 || (AE == 1 && BK == 128), "MXFP8 rows: 128 codes (one line) per stage");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wavefront tile is a multiple of 32 x 32");
  static_assert(A_LOADS * RPL * WAVES == BM, "load split");
};

// epilogues that pair W1 and W3 blocks (silu(W1 x) * W3 x)
__host__ __device__ constexpr bool is_swiglu(int epi) {
  return epi == EPI_SWIGLU || epi == EPI_SWIGLU_MX8;
}

// weight storage of the grouped GEMM's second operand
// kWMx4A8: MXFP4 weights with MXFP8 token rows (the scaled f8f6f4 MFMA)
constexpr int kWBf16 = 0, kWFp8 = 1, kWMxfp4 = 2, kWMx4A8 = 3;

// LDS geometry of a shape with bf16, E4M3 or MXFP4 weights
template <class SH, int WQ>
struct Geo {
  static constexpr bool MX4 = WQ == kWMxfp4 || WQ == kWMx4A8;  // E2M1 weights, E8M0 scales
  static constexpr bool A8 = WQ == kWMx4A8;                      // E4M3 token rows
  static_assert(A8 == (SH::AE == 1), "MXFP8 token rows go with the 1-byte tile shapes");
  static constexpr int B_ROWB = WQ == kWBf16 ? SH::ROWB : WQ == kWFp8 ? SH::BK : SH::BK / 2;
  static constexpr int B_CH = B_ROWB / 16;            // its 16-byte chunks
  static constexpr int B_RPL = 1024 / B_ROWB;         // weight rows one 1 KB load covers
  static constexpr int B_LOADS = SH::BN / B_RPL / SH::WAVES;
  // MXFP4: the stage's E8M0 scales, one dword (BK / 32 = 4 blocks) per weight row, loaded 32
  // rows per wavefront load into 256-byte areas (the other 32 lanes carry no address)
  static constexpr int SC_LOADS = MX4 ? SH::BN / 32 / SH::WAVES : 0;
  static constexpr int SC_BYTES = MX4 ? SH::BN / 32 * 256 : 0;
  // MXFP8 token rows: the stage's E8M0 scales, one dword (BK / 32 = 4 blocks) per row, 32 rows
  // per load into 256-byte areas; every wavefront issues the same count (areas past the tile's
  // rows take zeros), so the wait counts stay uniform
  static constexpr int A_SC_LOADS = A8 ? (SH::BM / 32 + SH::WAVES - 1) / SH::WAVES : 0;
  static constexpr int A_SC_BYTES = A_SC_LOADS * SH::WAVES * 256;
  static constexpr int LA = SH::A_LOADS + A_SC_LOADS;    // token-row loads per wavefront
  static constexpr int LB = B_LOADS + SC_LOADS;          // weight-side loads per wavefront
  static constexpr int L = LA + LB;                      // loads per wavefront per stage
  static constexpr int A_STAGE = SH::A_BYTES + A_SC_BYTES;
  static constexpr int B_STAGE = SH::BN * B_ROWB + SC_BYTES;
  static_assert(!MX4 || (SH::BK == 128 && SC_LOADS * 32 * SH::WAVES == SH::BN),
                "MXFP4 stages hold 128 k: one scale dword per row");
  static_assert(!A8 || A_SC_LOADS * 32 * SH::WAVES >= SH::BM, "MXFP8 scale loads");
  // MFMA sub-steps per stage: 16 k (bf16 32x32x16) or 64 k (scaled f8f6f4 32x32x64)
  static constexpr int KSUB = A8 ? SH::BK / 64 : SH::KK;
  // LDS: S slots of the token-row tile, then SB slots of the weight tile
  static constexpr int LDS = SH::S * A_STAGE + SH::SB * B_STAGE;
  static_assert(B_LOADS * B_RPL * SH::WAVES == SH::BN, "load split");
  // Each barrier issues the operand with fewer stages first (its step is needed sooner).  WAIT:
  // the loads a wavefront issued after the token rows and weights of step lk + 1, when step lk
  // waits for them (only loads are in flight inside the k-loop).  PRO_WAIT: the wait for step 0
  // at the start of a tile; the previous tile's stores were issued after the prologue, so with
  // S != SB it waits for everything rather than count on loads and stores completing in order.
  static constexpr int WAIT = SH::S == SH::SB ? (SH::S - 2) * L
                              : SH::S < SH::SB ? LB : LA;
  static constexpr int PRO_WAIT = SH::S == SH::SB ? (SH::S - 2) * L : 0;
  static_assert(SH::S >= 2 && WAIT < 64 && PRO_WAIT < 64, "loads in flight fit the vmcnt counter");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

using PrefillShape = TileShape<256, 256, 2, 4, 2, 64, 3>;
using DecodeShape = TileShape<32, 256, 1, 4, 4>;
// FP8 weights halve the weight tile.  Decode: stages of 128 k (each weight row a whole 128-byte
// line; with 64 k every line was fetched in two halves a k-step apart), two of them so that two
// workgroups fit per CU (eight wavefronts with loads in flight).  Measured on the DeepSeek-shaped
// gate-up: 1.35 ms, against 1.51 ms with 64-k stages (three, two workgroups), 1.86 ms with three
// 128-k stages (one workgroup) and 2.09 ms with seven 64-k stages (one workgroup).  The 64-k
// shape serves K not divisible by 128.  Prefill: two 64-k stages, as for bf16.
using PrefillShapeFp8 = TileShape<256, 256, 2, 4, 2>;
using DecodeShapeFp8 = TileShape<32, 256, 1, 4, 3>;
using DecodeShapeFp8K128 = TileShape<32, 256, 1, 4, 2, 128>;
// MXFP4: 128-k stages (64-byte code rows, one scale dword per row), two of them (52 KB) so that
// three workgroups fit per CU: a tile streams a quarter of the bf16 bytes, so its start and end
// weigh more, and a third workgroup keeps the CU's loads going through them (DeepSeek-shaped
// decode layer 1.26 -> 1.19 ms against three stages and two workgroups); every group size runs
// on this 32-row shape
using ShapeMxfp4 = TileShape<32, 256, 1, 4, 2, 128>;
// MXFP8 token rows with MXFP4 weights: the same 32-row blocking and two stages; a stage's token
// rows are one 128-byte line each (128 E4M3 codes) plus a scale dword (46 KB for both stages)
using ShapeMx4A8 = TileShape<32, 256, 1, 4, 2, 128, 2, 1>;
// ... and for groups of >= 128 rows on average, 256 x 256 tiles with two stages of the token
// rows (34 KB each) and three of the weights (18 KB each).  Wavefront tiles of 64 token rows x 128 columns: per 64-k MFMA step a
// token block takes two 16-byte LDS reads per lane and a weight block one, so four weight blocks
// and two token blocks (10 reads for 8 MFMAs) beat the 128 x 64 split of the bf16 shape
using PrefillShapeMx4A8 = TileShape<256, 256, 4, 2, 2, 128, 3, 1>;

// ---- tile bookkeeping shared by the GEMM and its tail reduction ---------------------------------

struct TileLoc {
  int row_base, m0, rows_here, n_t, g;
  int w;  // index of the group's weights in b / b2 / the scales (its slot when group_slot is set)
};

// An int32 at a uniform index of a table that earlier kernels wrote (the tile map, the group
// offsets, the expert -> slot table): a scalar load through the scalar cache, which keeps the
// tile-to-tile lookups off the vector-memory path (whose loads would each wait for every load
// and store in flight) and, after the first tile, hits in the scalar cache.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* a, int i) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  return ((cptr)a)[__builtin_amdgcn_readfirstlane(i)];
}

// tile `tile` of the (unsplit) tile list: its group, row block and column block
template <class SH, int GN>
__device__ __forceinline__ TileLoc locate_tile(const GroupedGemm& p, int tile) {
  int g = 0, row_base = 0, rows = p.static_rows, li = tile;
  tile = __builtin_amdgcn_readfirstlane(tile);
  if (p.tile_info) {
    // the tile map's own entry for this tile: one 16-byte scalar load (the search below costs a
    // dependent load per halving of the groups)
    typedef const __attribute__((address_space(4))) i32x4* cptr4;
    const i32x4 e = ((cptr4)p.tile_info)[tile];
    g = e[0];
    li = tile - e[1];
    row_base = e[2];
    rows = e[3];
  } else if (p.tile_start) {
    int lo = 0, hi2 = p.G;  // largest g with tile_start[g] <= tile
    while (hi2 - lo > 1) {
      const int mid = (lo + hi2) >> 1;
      if (ld_uniform(p.tile_start, mid) <= tile) lo = mid;
      else hi2 = mid;
    }
    g = lo;
    li = tile - ld_uniform(p.tile_start, g);
    row_base = ld_uniform(p.offsets, g);
    rows = ld_uniform(p.offsets, g + 1) - row_base;
  }
  const int mt = (rows + SH::BM - 1) / SH::BM;
  const int nblk = li / (mt * GN), rem = li % (mt * GN);
  TileLoc t;
  t.g = g;
  // a slot of -1 would mean a group with rows whose weights are not resident; the caller rules
  // that out, and slot 0 keeps the address in range if it ever happened
  t.w = p.group_slot && g < p.G_routed ? max(ld_uniform(p.group_slot, g), 0) : g;
  t.row_base = row_base;
  // the group's 32-row blocks are spread evenly over its mt row tiles (each gets at most BM / 32
  // of them, since mt = ceil(blocks / (BM / 32))), so no tile is a nearly empty remainder and
  // the MFMAs of blocks past a tile's rows can be skipped without some tiles finishing far ahead
  const int nb = (rows + 31) / 32, r = rem % mt;
  const int b0 = (int)((int64_t)r * nb / mt), b1 = (int)((int64_t)(r + 1) * nb / mt);
  t.m0 = b0 * 32;
  t.n_t = nblk * GN + rem / mt;
  t.rows_here = min((b1 - b0) * 32, rows - t.m0);
  return t;
}

// XCD x takes tiles [lo, lo + n) of the list, nx workgroups at a time.  When the last round is
// at most half full and a tail buffer is given, each of its `tail` tiles is cut into `pieces`
// k-ranges so the round's workgroups stay busy; the GEMM then has full * nx + tail * pieces
// work items in this XCD.
struct TailPlan {
  int lo, n, full, tail, pieces;
};
__device__ __forceinline__ TailPlan tail_plan(int total, int xcd, int nx, int kt, bool enabled) {
  const int per_xcd = (total + 7) / 8;
  TailPlan t;
  t.lo = xcd * per_xcd;
  t.n = max(0, min(per_xcd, total - t.lo));
  t.full = t.n / nx;
  t.tail = t.n - t.full * nx;
  t.pieces = 1;
  if (enabled && t.tail > 0 && 2 * t.tail <= nx) {
    int ks = min(4, nx / t.tail);
    while (ks > 1 && (kt / ks < 8 || t.tail * ks > kTailPieces)) --ks;
    t.pieces = ks;
  }
  return t;
}

// The epilogue: lane holds token l32 of block i and columns 8q + 4hi + (0..3) of each
// 32-column block j (the weights were the MFMA's first operand: D[column][token]).  With FP8
// weights each column's accumulator is first multiplied by its weight row's scale.
template <class SH, int EPI, int WQ>
__device__ __forceinline__ void store_tile(const GroupedGemm& p, const TileLoc& t, int ks,
                                           const f32x16 (&acc)[SH::TM][SH::TN], int wm, int wn,
                                           int l32, int hi, int i_only = -1) {
  constexpr int BN = SH::BN, TM = SH::TM, TN = SH::TN;
  const int64_t out_row0 = (int64_t)t.row_base + t.m0;
  // per-column scales of this tile (1 for bf16 weights), loaded once for all token blocks
  float4 sc[TN][4];
  if constexpr (WQ == kWFp8) {
    const bool extra = p.tile_start && t.g >= p.G_routed;
    const float* s1 = extra ? p.b_scale_extra : p.b_scale + (int64_t)t.w * p.N;
    const float* s2 = !is_swiglu(EPI) ? s1
                      : extra ? p.b2_scale_extra : p.b2_scale + (int64_t)t.w * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // SwiGLU: blocks j (W1) and j + 1 (W3) hold the same 32 columns
        const int col = is_swiglu(EPI)
                            ? t.n_t * (BN / 2) + wn * (SH::WTN / 2) + (j / 2) * 32 + 8 * q + 4 * hi
                            : t.n_t * BN + wn * SH::WTN + j * 32 + 8 * q + 4 * hi;
        const float* src = (is_swiglu(EPI) && (j & 1)) ? s2 : s1;
        sc[j][q] = col < p.N ? *(const float4*)(src + col) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
  }
  auto scaled = [&](int i, int j, int q, int e) -> float {
    if constexpr (WQ == kWFp8) {
      const float4 v = sc[j][q];
      const float f = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
      return acc[i][j][4 * q + e] * f;
    } else {
      return acc[i][j][4 * q + e];
    }
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i_only >= 0 && i != i_only) continue;
    const int tok = wm * SH::WTM + i * 32 + l32;
    if (tok >= t.rows_here) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      uint16_t* crow = (uint16_t*)p.c + (out_row0 + tok) * p.ldc;
      // blocks j (W1) and j + 1 (W3) hold the same 32 columns
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int col0 = t.n_t * (BN / 2) + wn * (SH::WTN / 2) + (j / 2) * 32;
        if (col0 + 32 <= p.N) {  // a whole block (the lane pair of the token row agrees)
          uint32_t d[4][2];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = silu_fast(scaled(i, j, q, e)) * scaled(i, j + 1, q, e);
            d[q][0] = pack_bf16x2(h[0], h[1]);
            d[q][1] = pack_bf16x2(h[2], h[3]);
          }
#pragma unroll
          for (int q = 0; q < 4; q += 2)
            *(uint4*)(crow + col0 + 8 * q + 8 * hi) = swap_halves(d[q][0], d[q][1], d[q + 1][0], d[q + 1][1]);
          continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = t.n_t * (BN / 2) + wn * (SH::WTN / 2) + (j / 2) * 32 + 8 * q + 4 * hi;
          if (col < p.N) {
            float h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = silu_fast(scaled(i, j, q, e)) * scaled(i, j + 1, q, e);
            uint2 v;
            v.x = pack_bf16x2(h[0], h[1]);
            v.y = pack_bf16x2(h[2], h[3]);
            *(uint2*)(crow + col) = v;
          }
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU_MX8) {
      // MXFP8 output: a 32-column block of the activation row is one MX block, held half by
      // this lane and half by lane ^ 32 (the same token row), which share its largest magnitude
      uint8_t* crow = (uint8_t*)p.c + (out_row0 + tok) * p.ldc;
      uint8_t* srow = p.c_mx + (out_row0 + tok) * (p.N / 32);
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const int col0 = t.n_t * (BN / 2) + wn * (SH::WTN / 2) + (j / 2) * 32;
        if (col0 >= p.N) continue;  // N % 32 == 0: a block is all in or all out
        float h[16];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[4 * q + e] = silu_fast(scaled(i, j, q, e)) * scaled(i, j + 1, q, e);
            amax = fmaxf(amax, fabsf(h[4 * q + e]));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const uint32_t sc = mxfp8_scale_code(amax);
        uint32_t w[4];  // codes of columns 8q + 4hi .. + 3
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = mxfp8_pack4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3], sc);
        // lane half 0 trades its quads 2, 3 (columns 16 .., 24 ..) for half 1's quads 0, 1
        // (columns 4 .., 12 ..): half h then holds columns 16h .. 16h + 15, one 16-byte store
        const auto s02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        *(uint4*)(crow + col0 + 16 * hi) = make_uint4(s02[0], s02[1], s13[0], s13[1]);
        if (hi == 0) srow[col0 / 32] = (uint8_t)sc;
      }
    } else if constexpr (EPI == EPI_BF16) {
      uint16_t* crow = (uint16_t*)p.c + (out_row0 + tok) * p.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col0 = t.n_t * BN + wn * SH::WTN + j * 32;
        if (col0 + 32 <= p.N) {  // a whole block (the lane pair of the token row agrees)
#pragma unroll
          for (int q = 0; q < 4; q += 2)
            *(uint4*)(crow + col0 + 8 * q + 8 * hi) = swap_halves(
                pack_bf16x2(scaled(i, j, q, 0), scaled(i, j, q, 1)),
                pack_bf16x2(scaled(i, j, q, 2), scaled(i, j, q, 3)),
                pack_bf16x2(scaled(i, j, q + 1, 0), scaled(i, j, q + 1, 1)),
                pack_bf16x2(scaled(i, j, q + 1, 2), scaled(i, j, q + 1, 3)));
          continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = t.n_t * BN + wn * SH::WTN + j * 32 + 8 * q + 4 * hi;
          if (col < p.N) {
            uint2 v;
            v.x = pack_bf16x2(scaled(i, j, q, 0), scaled(i, j, q, 1));
            v.y = pack_bf16x2(scaled(i, j, q, 2), scaled(i, j, q, 3));
            *(uint2*)(crow + col) = v;
          }
        }
      }
    } else {
      float* crow = (float*)p.c + ks * p.c_split_stride + (out_row0 + tok) * p.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = t.n_t * BN + wn * SH::WTN + j * 32 + 8 * q + 4 * hi;
          if (col + 3 < p.N && (p.ldc & 3) == 0) {
            *(float4*)(crow + col) = make_float4(scaled(i, j, q, 0), scaled(i, j, q, 1),
                                                 scaled(i, j, q, 2), scaled(i, j, q, 3));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < p.N) crow[col + e] = scaled(i, j, q, e);
          }
        }
    }
  }
}

// fp32 partial tile `slot` of XCD `xcd` in the tail buffer, laid out [block i][block j][quad]
// [thread][4]: a thread moves 16 bytes at a time and a wavefront 1 KB contiguous runs
template <class SH>
__device__ __forceinline__ float4* tail_slot(const GroupedGemm& p, int xcd, int slot) {
  constexpr int64_t kRegs = SH::TM * SH::TN * 16;
  return (float4*)(p.tail_part + ((int64_t)xcd * kTailPieces + slot) * kRegs * SH::THREADS);
}

template <class SH, int EPI, bool GATHER, int GN, int WQ>
__global__ __launch_bounds__(SH::THREADS) void gemm_kernel(GroupedGemm p) {
  using GE = Geo<SH, WQ>;
  constexpr int BM = SH::BM, BN = SH::BN, WN = SH::WN, S = SH::S, SB = SH::SB, L = GE::L;
  constexpr int TM = SH::TM, TN = SH::TN, KK = GE::KSUB, RPL = SH::RPL;
  constexpr int A_STAGE = GE::A_STAGE, A_SC_LOADS = GE::A_SC_LOADS;
  constexpr int B_ROWB = GE::B_ROWB, B_RPL = GE::B_RPL, B_LOADS = GE::B_LOADS, B_CH = GE::B_CH;
  constexpr int ROWB = SH::ROWB, CH = SH::CH;
  constexpr int SC_LOADS = GE::SC_LOADS, B_STAGE = GE::B_STAGE;
  constexpr int SC_OFF = SH::BN * GE::B_ROWB;  // scale tile in a weight stage
  static_assert(!is_swiglu(EPI) || TN % 2 == 0, "SwiGLU pairs W1 and W3 blocks");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid / WN, wn = wid % WN;
  const int K = p.K, KT = K / SH::BK;
  const int NT = is_swiglu(EPI) ? (p.N + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  const int total_base =
      p.tile_start ? ld_uniform(p.tile_start, p.G) : (p.static_rows + BM - 1) / BM * NT;
  // split-K: ksplit consecutive copies of the tile list; copy ks reduces over its share of the
  // k-steps into the partial output c + ks * c_split_stride
  const int ks_n = p.ksplit > 1 ? p.ksplit : 1;
  const int nx = gridDim.x / 8, xcd = blockIdx.x % 8;
  const TailPlan plan = tail_plan(total_base * ks_n, xcd, nx, KT, p.tail_part && ks_n == 1);
  const int items = plan.pieces > 1 ? plan.full * nx + plan.tail * plan.pieces : plan.n;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.a, (uint32_t)(p.a_rows * K * SH::AE));
  // MXFP8 token rows: their E8M0 scales, row-major [a_rows, K / 32]
  const __amdgpu_buffer_rsrc_t rAS = make_rsrc(GE::A8 ? (const void*)p.a_mx : p.a,
                                               GE::A8 ? (uint32_t)(p.a_rows * (K / 32)) : 0u);

  const int l32 = lane & 31, hi = lane >> 5;
  const int sw = row_swizzle<CH>(l32), swb = row_swizzle<B_CH>(l32);
  const uint32_t a_frag = (uint32_t)((wm * SH::WTM + l32) * ROWB);
  const uint32_t b_frag = (uint32_t)((wn * SH::WTN + l32) * B_ROWB);
  char* const a_slots = smem;                      // S slots of A_BYTES
  char* const b_slots = smem + S * A_STAGE;        // SB slots of B_STAGE

  struct Tile {
    TileLoc loc;
    int kt0, ktn, ks, slot;  // slot >= 0: a piece of a split tail tile, partial goes there
  };
  auto locate = [&](int it, Tile& t) -> bool {
    if (it >= items) return false;
    int tile_all = plan.lo + it, kt0 = 0, ktn = KT, slot = -1;
    if (plan.pieces > 1 && it >= plan.full * nx) {
      const int j = it - plan.full * nx, piece = j % plan.pieces;
      tile_all = plan.lo + plan.full * nx + j / plan.pieces;
      kt0 = (int)((int64_t)piece * KT / plan.pieces);
      ktn = (int)((int64_t)(piece + 1) * KT / plan.pieces) - kt0;
      slot = j;
    }
    const int ks = tile_all / total_base, tile = tile_all - ks * total_base;
    if (ks_n > 1) {
      kt0 = (int)((int64_t)ks * KT / ks_n);
      ktn = (int)((int64_t)(ks + 1) * KT / ks_n) - kt0;
    }
    t.loc = locate_tile<SH, GN>(p, tile);
    t.ks = ks;
    t.kt0 = kt0;
    t.ktn = ktn;
    t.slot = slot;
    return true;
  };

  // per-lane source offsets of the current tile's loads (lane: row lane / 8, chunk lane % 8)
  uint32_t a_off[SH::A_LOADS], b_off[B_LOADS];
  uint32_t s_off[SC_LOADS > 0 ? SC_LOADS : 1];
  uint32_t as_off[A_SC_LOADS > 0 ? A_SC_LOADS : 1];
  __amdgpu_buffer_rsrc_t rB, rB2, rS, rS2;
  int kt0 = 0, ktn = 0;
  auto setup = [&](const Tile& t) {
    // uniform, but the 64-bit divisions that split k leave them in VGPRs; a VGPR soffset would
    // make every buffer load a readfirstlane loop
    kt0 = __builtin_amdgcn_readfirstlane(t.kt0);
    ktn = __builtin_amdgcn_readfirstlane(t.ktn);
    const bool extra = p.tile_start && t.loc.g >= p.G_routed;
    const int wsel = __builtin_amdgcn_readfirstlane(t.loc.w);  // uniform: keeps the rsrc scalar
    // bytes of one weight row and of one group's matrix
    const int64_t wrow = WQ == kWBf16 ? 2LL * K : WQ == kWFp8 ? (int64_t)K : (int64_t)K / 2;
    const int64_t gbytes = WQ == kWBf16 ? p.b_stride * 2 : WQ == kWFp8 ? p.b_stride : p.b_stride / 2;
    const char* bbase =
        (const char*)(extra ? p.b_extra : p.b) + (extra ? 0 : (int64_t)wsel * gbytes);
    const char* b2base = bbase;
    if (is_swiglu(EPI))
      b2base = (const char*)(extra ? p.b2_extra : p.b2) + (extra ? 0 : (int64_t)wsel * gbytes);
    const uint32_t b_bytes = (uint32_t)((int64_t)p.N * wrow);
    rB = make_rsrc(bbase, b_bytes);
    rB2 = make_rsrc(b2base, b_bytes);
    if constexpr (GE::MX4) {
      // scales blocked by 32 rows: the dword of row r for 128-k step kt at
      // ((r / 32) * KT + kt) * 128 + (r % 32) * 4, so a block's 32 dwords are one line
      const int64_t sgroup = (int64_t)p.N * (K / 32);
      const uint8_t* sbase = extra ? p.b_mx_extra : p.b_mx + (int64_t)wsel * sgroup;
      const uint8_t* s2base = sbase;
      if (is_swiglu(EPI)) s2base = extra ? p.b2_mx_extra : p.b2_mx + (int64_t)wsel * sgroup;
      rS = make_rsrc(sbase, (uint32_t)sgroup);
      rS2 = make_rsrc(s2base, (uint32_t)sgroup);
#pragma unroll
      for (int i = 0; i < SC_LOADS; ++i) {
        const int n = (wid * SC_LOADS + i) * 32 + lane;  // lanes 32..63 load nothing
        const int src = is_swiglu(EPI) ? t.loc.n_t * (BN / 2) + (n >> 6) * 32 + (n & 31) : t.loc.n_t * BN + n;
        s_off[i] = lane < 32 && src < p.N ? (uint32_t)((src >> 5) * KT * 128 + (src & 31) * 4)
                                          : kOutOfRange;
      }
    }
    // the gathered row indices are read for every lane (rows past the tile's end read its last
    // row and are masked afterwards), so the loads go out together and are waited for once
    int a_src[SH::A_LOADS];
#pragma unroll
    for (int i = 0; i < SH::A_LOADS; ++i) {
      const int r = (wid * SH::A_LOADS + i) * RPL + lane / CH;
      const int prow = t.loc.row_base + t.loc.m0 + min(r, t.loc.rows_here - 1);
      a_src[i] = GATHER ? p.row_map[prow] : prow;
    }
#pragma unroll
    for (int i = 0; i < SH::A_LOADS; ++i) {
      const int r = (wid * SH::A_LOADS + i) * RPL + lane / CH;
      const int c = (lane % CH) ^ row_swizzle<CH>(r);
      a_off[i] = r < t.loc.rows_here ? (uint32_t)((int64_t)a_src[i] * K * SH::AE) + c * 16 : kOutOfRange;
    }
    if constexpr (GE::A8) {
      // the scale dword of tile row r for step kt sits at row * (K / 32) + kt * 4; lanes
      // 32..63 and rows past the tile load nothing
#pragma unroll
      for (int i = 0; i < A_SC_LOADS; ++i) {
        const int r = (wid * A_SC_LOADS + i) * 32 + l32;
        const int prow = t.loc.row_base + t.loc.m0 + min(r, t.loc.rows_here - 1);
        const int src = GATHER ? p.row_map[prow] : prow;
        as_off[i] = lane < 32 && r < t.loc.rows_here ? (uint32_t)src * (uint32_t)(K / 32) : kOutOfRange;
      }
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      // lane: weight row lane / (chunks per row), chunk lane % (chunks per row)
      const int n = (wid * B_LOADS + i) * B_RPL + lane / B_CH;
      const int c = (lane % B_CH) ^ row_swizzle<B_CH>(n);
      const int src = is_swiglu(EPI) ? t.loc.n_t * (BN / 2) + (n >> 6) * 32 + (n & 31) : t.loc.n_t * BN + n;
      // MXFP4 codes are blocked: row r's 64 bytes of 128-k step kt at ((r / 32) * KT + kt) * 2048
      // + (r % 32) * 64
      const uint32_t row_at = GE::MX4 ? (uint32_t)((src >> 5) * KT * 2048 + (src & 31) * 64)
                                            : (uint32_t)(src * wrow);
      b_off[i] = src < p.N ? row_at + c * 16 : kOutOfRange;
    }
  };
  // local k-step lk of the current tile into LDS slots `slot` (token rows) and `bslot` (weights);
  // lk >= ktn loads nothing.  The 256 x 256 MXFP8 tiles instead re-read the tile's last k-step
  // there (into a slot nothing reads before the next tile's loads): with the masked form the
  // compiler turned the offset selects into branches inside their k-loop, splitting the region
  // the MFMAs and fragment reads are scheduled in (the re-read is 4 % more bytes per tile; the
  // Qwen3-shaped layer on MXFP4 weights went from 1.57 to 1.51 ms).  The 32-row tiles stream
  // weights, where the extra bytes cost more than the branches (1 % on the decode gate-up).
  constexpr bool REREAD = GE::A8 && TM * TN >= 8;
  auto issue_a = [&](int lk, int slot) {
    const bool valid = REREAD || lk < ktn;
    if constexpr (REREAD) lk = lk < ktn ? lk : ktn - 1;
    char* sa = a_slots + slot * A_STAGE;
    const int kb = valid ? (kt0 + lk) * ROWB : 0;
#pragma unroll
    for (int i = 0; i < SH::A_LOADS; ++i)
      load_lds16(rA, sa + (wid * SH::A_LOADS + i) * 1024, valid ? a_off[i] : kOutOfRange, kb);
    if constexpr (GE::A8) {
      // the stage's 4 scale bytes of each row (k-blocks (kt0 + lk) * 4 .. + 3)
      const int kbs = valid ? (kt0 + lk) * 4 : 0;
#pragma unroll
      for (int i = 0; i < A_SC_LOADS; ++i)
        load_lds4(rAS, sa + SH::A_BYTES + (wid * A_SC_LOADS + i) * 256,
                  valid ? as_off[i] : kOutOfRange, kbs);
    }
  };
  auto issue_b = [&](int lk, int bslot) {
    const bool valid = REREAD || lk < ktn;
    if constexpr (REREAD) lk = lk < ktn ? lk : ktn - 1;
    char* sb = b_slots + bslot * B_STAGE;
    const int kbw = valid ? (kt0 + lk) * (GE::MX4 ? 32 * B_ROWB : B_ROWB) : 0;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int blk = wid * B_LOADS + i;
      const bool second = is_swiglu(EPI) && (((blk * B_RPL) >> 5) & 1);
      load_lds16(second ? rB2 : rB, sb + blk * 1024, valid ? b_off[i] : kOutOfRange, kbw);
    }
    if constexpr (GE::MX4) {
      // the stage's 4 scale bytes of each row (k-blocks (kt0 + lk) * 4 .. + 3)
      const int kbs = valid ? (kt0 + lk) * 128 : 0;
#pragma unroll
      for (int i = 0; i < SC_LOADS; ++i) {
        const int blk = wid * SC_LOADS + i;
        const bool second = is_swiglu(EPI) && (blk & 1);
        load_lds4(second ? rS2 : rS, sb + SC_OFF + blk * 256, valid ? s_off[i] : kOutOfRange, kbs);
      }
    }
  };
  // weight-side loads [i0, i1) of step lk into slot bslot: the weight tile's B_LOADS, then (E2M1
  // weights) its SC_LOADS scale loads
  auto issue_b_part = [&](int lk, int bslot, int i0, int i1) {
    const bool valid = REREAD || lk < ktn;
    if constexpr (REREAD) lk = lk < ktn ? lk : ktn - 1;
    char* sb = b_slots + bslot * B_STAGE;
    const int kbw = valid ? (kt0 + lk) * (GE::MX4 ? 32 * B_ROWB : B_ROWB) : 0;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      if (i < i0 || i >= i1) continue;
      const int blk = wid * B_LOADS + i;
      const bool second = is_swiglu(EPI) && (((blk * B_RPL) >> 5) & 1);
      load_lds16(second ? rB2 : rB, sb + blk * 1024, valid ? b_off[i] : kOutOfRange, kbw);
    }
    if constexpr (GE::MX4) {
      const int kbs = valid ? (kt0 + lk) * 128 : 0;
#pragma unroll
      for (int i = 0; i < SC_LOADS; ++i) {
        if (B_LOADS + i < i0 || B_LOADS + i >= i1) continue;
        const int blk = wid * SC_LOADS + i;
        const bool second = is_swiglu(EPI) && (blk & 1);
        load_lds4(second ? rS2 : rS, sb + SC_OFF + blk * 256, valid ? s_off[i] : kOutOfRange, kbs);
      }
    }
  };
  // The step-lk barrier sends out the token rows of step lk + S and (with S == SB) the weights of
  // step lk + SB, the shallower operand first; the start of the k-loop sends steps S - 1 and
  // SB - 1 in the same order, so the wait at every barrier is the constant GE::WAIT.
  auto issue_both = [&](int la, int sa, int lb, int sb) {
    if constexpr (S <= SB) {
      issue_a(la, sa);
      issue_b(lb, sb);
    } else {
      issue_b(lb, sb);
      issue_a(la, sa);
    }
  };
  auto prologue = [&]() {  // steps 0 .. S - 2 (token rows) and 0 .. SB - 2 (weights), by step
#pragma unroll
    for (int s = 0; s < (S > SB ? S : SB) - 1; ++s) {
      if (s < S - 1) issue_a(s, s);
      if (s < SB - 1) issue_b(s, s);
    }
  };

  f32x16 acc[TM][TN];
  bf16x8 fa[2][TM], fb[2][TN];
  // MXFP8 x MXFP4: 32 E4M3 codes per token lane, 32 E2M1 codes per weight lane, and the E8M0
  // scale of the lane's k-block (lane half hi supplies block hi of the MFMA's 64 k)
  i32x8 fa8[2][TM];
  i32x4 fb4[2][TN];
  int sca[2][TM], scb[2][TN];
  // NV: the wavefront's token blocks that hold rows of the tile (the others are skipped)
  auto read_frags = [&](auto nv, const char* sta, const char* st, int kk, int buf) {
    constexpr int NV = decltype(nv)::value;
    if constexpr (GE::A8) {
      // sub-step kk covers k 64kk .. 64kk + 63 of the stage.  Token lane: k 64kk + 16hi .. + 15
      // (chunk 4kk + hi of the 128-byte row) then k 64kk + 32 + 16hi .. + 15 (chunk 4kk + 2 +
      // hi).  Weight lane: k 64kk + 32hi .. + 31 (chunk 2kk + hi of the 64-byte row).  Both take
      // the scale of k-block 2kk + hi, byte 2kk + hi of the row's scale dword.
      const int blk = 2 * kk + hi;
      const uint32_t c0 = (uint32_t)(((4 * kk + hi) ^ sw) * 16);
      const uint32_t c1 = (uint32_t)(((4 * kk + 2 + hi) ^ sw) * 16);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const char* ra = sta + a_frag + i * 32 * ROWB;
        const i32x4 lo = *(const i32x4*)(ra + c0), up = *(const i32x4*)(ra + c1);
        fa8[buf][i] = i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        const uint32_t s4 =
            *(const uint32_t*)(sta + SH::A_BYTES + ((wm * SH::WTM) / 32 + i) * 256 + l32 * 4);
        sca[buf][i] = (int)((s4 >> (8 * blk)) & 0xffu);
      }
      const uint32_t woff = (uint32_t)((blk ^ swb) * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        fb4[buf][j] = *(const i32x4*)(st + b_frag + woff + j * 32 * B_ROWB);
        const uint32_t s4 =
            *(const uint32_t*)(st + SC_OFF + ((wn * SH::WTN) / 32 + j) * 256 + l32 * 4);
        scb[buf][j] = (int)((s4 >> (8 * blk)) & 0xffu);
      }
    } else {
      const uint32_t coff = (uint32_t)(((kk * 2 + hi) ^ sw) * 16);
#pragma unroll
      for (int i = 0; i < NV; ++i) fa[buf][i] = *(const bf16x8*)(sta + a_frag + coff + i * 32 * ROWB);
      if constexpr (GE::MX4) {
        // a k-sub's 16 codes are half of chunk kk / 2 of the 64-byte row; the lane takes 8 of them
        // (one dword) and the scale of their 32-block kk / 2
        const uint32_t woff = (uint32_t)((((kk >> 1) ^ swb) * 16) + (kk & 1) * 8 + hi * 4);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const uint32_t codes = *(const uint32_t*)(st + b_frag + woff + j * 32 * B_ROWB);
          const uint32_t sc4 =
              *(const uint32_t*)(st + SC_OFF + ((wn * SH::WTN) / 32 + j) * 256 + l32 * 4);
          const float scale = __uint_as_float(((sc4 >> (8 * (kk >> 1))) & 0xffu) << 23);
          fb[buf][j] = fp4x8_to_bf16(codes, scale);
        }
      } else if constexpr (WQ == kWFp8) {
        // a k-sub's 16 codes are chunk kk of the row; the lane takes half of it
        const uint32_t woff = (uint32_t)(((kk ^ swb) * 16) + hi * 8);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[buf][j] = fp8x8_to_bf16(*(const uint2*)(st + b_frag + woff + j * 32 * B_ROWB));
      } else {
        const uint32_t boff = (uint32_t)(((kk * 2 + hi) ^ swb) * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[buf][j] = *(const bf16x8*)(st + b_frag + boff + j * 32 * B_ROWB);
      }
    }
  };
  // weights as the first operand: D[column][token]
  auto mfmas = [&](auto nv, int buf) {
    constexpr int NV = decltype(nv)::value;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (GE::A8) {
          // v_mfma_scale_f32_32x32x64_f8f6f4: first operand E2M1 (format 4, registers 0-3),
          // second E4M3 (format 0), each with its lane's E8M0 scale
          const i32x4 w = fb4[buf][j];
          const i32x8 wa = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wa, fa8[buf][i], acc[i][j], 4, 0, 0, scb[buf][j], 0, sca[buf][i]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
        }
      }
  };
  // Every step issues L loads per wavefront (stage lk + S, masked past the end), so when step
  // lk waits for stage lk + 1 exactly S - 2 stages were issued after it.
  auto kloop = [&](auto nv) {
    constexpr int NV = decltype(nv)::value;
    read_frags(nv, a_slots, b_slots, 0, 0);
    issue_both(S - 1, S - 1, SB - 1, SB - 1);
    for (int lk = 0; lk < ktn; ++lk) {
      const char* cura = a_slots + (lk % S) * A_STAGE;
      const char* curb = b_slots + (lk % SB) * B_STAGE;
      const char* nxta = a_slots + ((lk + 1) % S) * A_STAGE;
      const char* nxtb = b_slots + ((lk + 1) % SB) * B_STAGE;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk < KK - 1) {
          read_frags(nv, cura, curb, kk + 1, (kk + 1) & 1);
        } else {
          wait_vmcnt<GE::WAIT>();  // step lk + 1 landed (this wavefront's share)
          wait_lgkmcnt<0>();       // this wavefront's reads of step lk returned
          barrier_keep_loads();    // ... and everyone else's
          read_frags(nv, nxta, nxtb, 0, 0);
          if constexpr (S < SB) issue_a(lk + S, lk % S);
          else issue_both(lk + S, lk % S, lk + SB, lk % SB);
        }
        // With a deeper weight ring (SB = S + 1) the weights of step lk + SB go out over the
        // first two sub-steps of step lk + 1, not at the barrier with the token rows: the loads
        // reach the L1 in a steadier stream (3 % faster on both prefill workloads than all of a
        // stage's loads issued in one sub-step; one load per two MFMAs was slower).  Step
        // lk + 1's barrier still waits for all but these (WAIT = LB).
        // (MXFP8 stages have two sub-steps, the second holding the barrier: all of the weight
        // stage goes out in the first, so that the barrier's wait count stays LB)
        constexpr int BSPAN = GE::A8 ? 1 : 2, BPER = (GE::LB + BSPAN - 1) / BSPAN;
        if constexpr (S < SB) {
          if (kk < BSPAN && lk > 0)
            issue_b_part(lk - 1 + SB, (lk - 1) % SB, kk * BPER, (kk + 1) * BPER);
        }
        mfmas(nv, kk & 1);
        if constexpr (GE::A8) {
          // few, long MFMAs per sub-step: the next sub-step's reads (3 per token block, 2 per
          // weight block) and the sub-step's global loads spread evenly over them
          constexpr int NM = NV * TN > 0 ? NV * TN : 1;
          constexpr int RD = (3 * NV + 2 * TN + NM - 1) / NM;
          constexpr int LDL = (S < SB ? GE::LA : L), LDB = S < SB ? GE::LB : 0;
#pragma unroll
          for (int m = 0; m < NV * TN; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
            if (kk == KK - 1) __builtin_amdgcn_sched_group_barrier(0x020, (LDL + NM - 1) / NM, 0);
            if (kk == 0 && LDB > 0) __builtin_amdgcn_sched_group_barrier(0x020, (LDB + NM - 1) / NM, 0);
          }
          continue;
        }
        // interleave: one MFMA, then one LDS read and one global load
#pragma unroll
        for (int m = 0; m < NV * TN; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (m < NV + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if constexpr (S < SB) {
            if ((kk == KK - 1 && m < SH::A_LOADS) ||
                (kk < BSPAN && m < BPER && kk * BPER + m < GE::LB))
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          } else {
            if (kk == KK - 1 && m < L) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
      }
    }
  };

  int it = blockIdx.x / 8;
  Tile cur;
  if (!locate(it, cur)) return;
  setup(cur);
  prologue();

  while (true) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    wait_vmcnt<GE::PRO_WAIT>();  // step 0 (and the previous tile's stores, issued after it)
    barrier_keep_loads();
    // token blocks of this wavefront that hold rows: the two wavefronts of a SIMD split the
    // tile's rows, so the SIMD's MFMA time follows the tile's real rows
    const int nv = __builtin_amdgcn_readfirstlane(
        min(TM, max(0, (cur.loc.rows_here - wm * SH::WTM + 31) / 32)));
    if constexpr (TM == 4) {
      if (nv == 4) kloop(std::integral_constant<int, 4>{});
      else if (nv == 3) kloop(std::integral_constant<int, 3>{});
      else if (nv == 2) kloop(std::integral_constant<int, 2>{});
      else if (nv == 1) kloop(std::integral_constant<int, 1>{});
      else kloop(std::integral_constant<int, 0>{});
    } else if constexpr (TM == 2 && GE::A8) {
      if (nv == 2) kloop(std::integral_constant<int, 2>{});
      else if (nv == 1) kloop(std::integral_constant<int, 1>{});
      else kloop(std::integral_constant<int, 0>{});
    } else {
      kloop(std::integral_constant<int, TM>{});
    }
    // everyone is done with the operand slots and the loads past the last stage have landed
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_keep_loads();

    const Tile done = cur;
    it += nx;
    const bool more = locate(it, cur);
    if (more) {  // the next tile's first stages load while this tile's results go out
      setup(cur);
      prologue();
    }

    if (done.slot >= 0) {
      // a piece of a split tail tile: park the fp32 partial for the tail reduction
      float4* dst = tail_slot<SH>(p, xcd, done.slot) + tid;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[((i * TN + j) * 4 + q) * SH::THREADS] =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    } else {
      store_tile<SH, EPI, WQ>(p, done.loc, done.ks, acc, wm, wn, l32, hi);
    }
    if (!more) break;
  }
}

// The split tail tiles: add each tile's fp32 partials in piece order, then the epilogue.  One
// workgroup per (XCD, tail tile, token block i), so the reduction spreads over many CUs.
template <class SH, int EPI, int GN, int WQ>
__global__ __launch_bounds__(SH::THREADS) void gemm_tail_kernel(GroupedGemm p, int nx) {
  constexpr int TM = SH::TM, TN = SH::TN;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wid / SH::WN, wn = wid % SH::WN;
  const int xcd = blockIdx.x % 8, t = (blockIdx.x / 8) % kTailPieces, ib = blockIdx.x / (8 * kTailPieces);
  const TailPlan plan = tail_plan(ld_uniform(p.tile_start, p.G), xcd, nx, p.K / SH::BK, true);
  if (plan.pieces <= 1 || t >= plan.tail) return;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i != ib) continue;
    for (int piece = 0; piece < plan.pieces; ++piece) {
      const float4* src = tail_slot<SH>(p, xcd, t * plan.pieces + piece) + tid;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = src[((i * TN + j) * 4 + q) * SH::THREADS];
          if (piece == 0) {
            acc[i][j][4 * q] = v.x;
            acc[i][j][4 * q + 1] = v.y;
            acc[i][j][4 * q + 2] = v.z;
            acc[i][j][4 * q + 3] = v.w;
          } else {
            acc[i][j][4 * q] += v.x;
            acc[i][j][4 * q + 1] += v.y;
            acc[i][j][4 * q + 2] += v.z;
            acc[i][j][4 * q + 3] += v.w;
          }
        }
    }
  }
  const TileLoc loc = locate_tile<SH, GN>(p, plan.lo + plan.full * nx + t);
  store_tile<SH, EPI, WQ>(p, loc, 0, acc, wm, wn, lane & 31, lane >> 5, ib);
}

template <class SH, int EPI, bool GATHER, int GN, int WQ = kWBf16>
static hipError_t run(const GroupedGemm& p, int max_tiles, int num_cus, hipStream_t s) {
  constexpr int LDS = Geo<SH, WQ>::LDS;
  auto kern = gemm_kernel<SH, EPI, GATHER, GN, WQ>;
  // the dynamic LDS size is raised once per device for each instantiation
  static std::atomic<uint64_t> lds_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? 1ull << dev : 0;
  if (!bit || !(lds_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    lds_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (max_tiles <= 0) return hipSuccess;
  // workgroups per CU: as many as the LDS holds, at most 8 wavefronts per CU (12 for the MXFP4
  // tiles, whose wavefronts need few enough registers for three per SIMD)
  int per_cu = (160 * 1024) / LDS;
  const int by_waves = (Geo<SH, WQ>::MX4 ? 12 : 8) / SH::WAVES;
  if (per_cu > by_waves) per_cu = by_waves;
  if (per_cu < 1) per_cu = 1;
  int grid = num_cus * per_cu;
  if (grid > max_tiles) grid = max_tiles;
  grid = (grid + 7) / 8 * 8;
  GroupedGemm q = p;
  if (!q.tile_start || q.ksplit > 1 || EPI == EPI_F32 || grid / 8 > kTailPieces) q.tail_part = nullptr;
  kern<<<grid, SH::THREADS, LDS, s>>>(q);
  e = hipGetLastError();
  if (e != hipSuccess || !q.tail_part) return e;
  gemm_tail_kernel<SH, EPI, GN, WQ><<<8 * kTailPieces * SH::TM, SH::THREADS, 0, s>>>(q, grid / 8);
  return hipGetLastError();
}

// Rows of a gate tile.  Every tile reads the whole [E, H] gate weight through LDS, so with
// 32-row tiles the weight's L2 -> LDS traffic is E / 32 times the tokens' (4x at 128 experts);
// 128-row tiles cut it to a quarter.  They are taken when the reduction is split (so that
// there are still enough workgroups) over many tokens and 64-128 experts.
int gemm_gate_bm(int T, int E, bool split) {
  return split && T >= 2048 && E > 32 && E <= 128 ? 128 : 32;
}

// choose tiles for a kind of GEMM from the rows a group holds on average (the gate: its tokens)
void gemm_bf16_tiling(GemmKind kind, int avg_rows_per_group, int N, int* bm, int* nt) {
  if (kind == GEMM_GATE) {
    const int bn = N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
    *bm = 32;
    *nt = (N + bn - 1) / bn;
    return;
  }
  const bool big = avg_rows_per_group >= kBigTileRows;
  *bm = big ? PrefillShape::BM : DecodeShape::BM;
  const int bn = big ? PrefillShape::BN : DecodeShape::BN;
  *nt = kind == GEMM_GATE_UP ? (N + bn / 2 - 1) / (bn / 2) : (N + bn - 1) / bn;
}

size_t gemm_tail_bytes(int avg_rows_per_group) {
  const bool big = avg_rows_per_group >= kBigTileRows;
  const size_t tile = big ? (size_t)PrefillShape::BM * PrefillShape::BN
                          : (size_t)DecodeShape::BM * DecodeShape::BN;
  return 8 * (size_t)kTailPieces * tile * sizeof(float);
}

hipError_t launch_gemm_bf16(GemmKind kind, const GroupedGemm& p, int avg_rows_per_group,
                            int num_cus, hipStream_t s) {
  int bm, nt;
  gemm_bf16_tiling(kind, avg_rows_per_group, p.N, &bm, &nt);
  if (p.ksplit > 1 && kind != GEMM_GATE) return hipErrorInvalidValue;  // fp32 output only
  if (p.a_mx && kind == GEMM_GATE) return hipErrorInvalidValue;
  if (kind == GEMM_GATE) bm = gemm_gate_bm(p.static_rows, p.N, p.ksplit > 1);
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
    if (bm == 128) {  // wavefront tiles of 64 tokens x 32 or 64 experts
      if (p.N <= 64) return run<TileShape<128, 64, 2, 2, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
      return run<TileShape<128, 128, 2, 2, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
    }
    if (p.N <= 32) return run<TileShape<32, 32, 1, 1, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 64) return run<TileShape<32, 64, 1, 2, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
    if (p.N <= 128) return run<TileShape<32, 128, 1, 4, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
    return run<TileShape<32, 256, 1, 4, 4>, EPI_F32, false, 1>(p, mt, num_cus, s);
  }
  const bool big = bm == PrefillShape::BM;
  const bool gather = p.row_map != nullptr;
  if (p.a_mx) {  // MXFP8 token rows: MXFP4 weights only
    if (!p.b_mx || p.K % 128 || (kind == GEMM_GATE_UP && (!p.b2_mx || !p.c_mx || p.N % 32)))
      return hipErrorInvalidValue;
    if (p.G > p.G_routed && (!p.b_mx_extra || (kind == GEMM_GATE_UP && !p.b2_mx_extra)))
      return hipErrorInvalidValue;
    if (gather && kind != GEMM_GATE_UP) return hipErrorInvalidValue;
    if (big) {
      using SH = PrefillShapeMx4A8;
      if (kind == GEMM_GATE_UP)
        return gather ? run<SH, EPI_SWIGLU_MX8, true, 8, kWMx4A8>(p, mt, num_cus, s)
                      : run<SH, EPI_SWIGLU_MX8, false, 8, kWMx4A8>(p, mt, num_cus, s);
      return run<SH, EPI_BF16, false, 8, kWMx4A8>(p, mt, num_cus, s);
    }
    if (kind == GEMM_GATE_UP)
      return gather ? run<ShapeMx4A8, EPI_SWIGLU_MX8, true, 1, kWMx4A8>(p, mt, num_cus, s)
                    : run<ShapeMx4A8, EPI_SWIGLU_MX8, false, 1, kWMx4A8>(p, mt, num_cus, s);
    return run<ShapeMx4A8, EPI_BF16, false, 1, kWMx4A8>(p, mt, num_cus, s);
  }
  if (p.b_mx) {  // MXFP4 weights: the 32-row shape for every group size, K % 128 == 0
    if (p.K % 128 || (kind == GEMM_GATE_UP && !p.b2_mx)) return hipErrorInvalidValue;
    if (p.G > p.G_routed && (!p.b_mx_extra || (kind == GEMM_GATE_UP && !p.b2_mx_extra)))
      return hipErrorInvalidValue;
    if (bm != ShapeMxfp4::BM) return hipErrorInvalidValue;  // tile map built for 32-row tiles
    if (kind == GEMM_GATE_UP)
      return gather ? run<ShapeMxfp4, EPI_SWIGLU, true, 1, kWMxfp4>(p, mt, num_cus, s)
                    : run<ShapeMxfp4, EPI_SWIGLU, false, 1, kWMxfp4>(p, mt, num_cus, s);
    return run<ShapeMxfp4, EPI_BF16, false, 1, kWMxfp4>(p, mt, num_cus, s);
  }
  if (p.b_scale) {  // FP8 weights
    if (kind == GEMM_GATE_UP && !p.b2_scale) return hipErrorInvalidValue;
    if (p.G > p.G_routed && (!p.b_scale_extra || (kind == GEMM_GATE_UP && !p.b2_scale_extra)))
      return hipErrorInvalidValue;
    if (kind == GEMM_GATE_UP) {
      if (big)
        return gather ? run<PrefillShapeFp8, EPI_SWIGLU, true, 8, kWFp8>(p, mt, num_cus, s)
                      : run<PrefillShapeFp8, EPI_SWIGLU, false, 8, kWFp8>(p, mt, num_cus, s);
      if (p.K % 128 == 0)
        return gather ? run<DecodeShapeFp8K128, EPI_SWIGLU, true, 1, kWFp8>(p, mt, num_cus, s)
                      : run<DecodeShapeFp8K128, EPI_SWIGLU, false, 1, kWFp8>(p, mt, num_cus, s);
      return gather ? run<DecodeShapeFp8, EPI_SWIGLU, true, 1, kWFp8>(p, mt, num_cus, s)
                    : run<DecodeShapeFp8, EPI_SWIGLU, false, 1, kWFp8>(p, mt, num_cus, s);
    }
    if (big) return run<PrefillShapeFp8, EPI_BF16, false, 8, kWFp8>(p, mt, num_cus, s);
    if (p.K % 128 == 0) return run<DecodeShapeFp8K128, EPI_BF16, false, 1, kWFp8>(p, mt, num_cus, s);
    return run<DecodeShapeFp8, EPI_BF16, false, 1, kWFp8>(p, mt, num_cus, s);
  }
  if (kind == GEMM_GATE_UP) {
    if (big)
      return gather ? run<PrefillShape, EPI_SWIGLU, true, 8>(p, mt, num_cus, s)
                    : run<PrefillShape, EPI_SWIGLU, false, 8>(p, mt, num_cus, s);
    return gather ? run<DecodeShape, EPI_SWIGLU, true, 1>(p, mt, num_cus, s)
                  : run<DecodeShape, EPI_SWIGLU, false, 1>(p, mt, num_cus, s);
  }
  if (big) return run<PrefillShape, EPI_BF16, false, 8>(p, mt, num_cus, s);
  return run<DecodeShape, EPI_BF16, false, 1>(p, mt, num_cus, s);
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
