// Internal declarations shared by the HIP sources of libmoe.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kSlotTile = 1024;    // routing slots handled by one permute block
constexpr int kMaxExperts = 1024;  // routed experts the routing kernels support
constexpr int kMaxDevices = 64;    // devices whose properties the host side caches
// rows of a group from which its bf16 expert GEMMs take the 256 x 256 tiles
constexpr int kBigTileRows = 128;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// MXFP8 (the OCP microscaling format with E4M3 elements and one E8M0 scale per 32 elements):
// the scale code of a block whose largest magnitude is amax: 2^(floor(log2 amax) - 8), the
// exponent clamped to [-126, 127] so that the scale is a normal float; 127 (scale 1) for a
// zero block.
__device__ __forceinline__ uint32_t mxfp8_scale_code(float amax) {
  if (!(amax > 0.f)) return 127u;
  // amax = m * 2^e with m in [0.5, 1): floor(log2(amax)) = e - 1
  int shared = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
  shared = shared < -126 ? -126 : (shared > 127 ? 127 : shared);
  return (uint32_t)(shared + 127);
}

// four values of a block with scale code sc -> four E4M3 codes in one dword (value 0 in the low
// byte).  The hardware conversion divides by the scale and rounds to nearest even, but turns
// quotients above the largest finite E4M3 value into NaN, so the values are first clamped to
// +-448 times the scale.
__device__ __forceinline__ uint32_t mxfp8_pack4(float a, float b, float c, float d, uint32_t sc) {
  typedef __attribute__((__vector_size__(2 * sizeof(short)))) short short2_t;
  const float scale = __uint_as_float(sc << 23), lim = 448.f * scale;
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  c = fminf(fmaxf(c, -lim), lim);
  d = fminf(fmaxf(d, -lim), lim);
  short2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Launchers (each returns hipGetLastError() of its launch(es)).
// ---------------------------------------------------------------------------

// route.hip: one wavefront per token; softmax, top-k, renormalise.  With `part` (a split gate's
// S partial sums, [S, T, E]) the logits are first summed from it, part 0 then 1 .. S - 1 as the
// split-K reduction adds them, and written to logits_out; else they are read from `logits`.
hipError_t launch_route(const float* logits, const float* bias, int T, int E, int k,
                        int renormalize, int bias_mode, int32_t* ids, float* w, hipStream_t s,
                        const float* part = nullptr, int S = 1, float* logits_out = nullptr);

// stats.hip: load statistics of the per-expert pick counts (raw, after launch_permute's scan)
// and the next balancing bias
hipError_t launch_load_stats(const int32_t* raw, int E, int capacity, void* stats,
                             float* bias_next, hipStream_t s);

// permute.hip
struct PermuteArgs {
  const int32_t* ids;      // [n] expert of each slot (slot = t*k + j)
  const uint8_t* inactive; // [n] or null: 1 = slot takes no part (already dropped)
  int n, k, E, T;
  int capacity;            // < 0 unlimited
  int ntiles;              // ceil(n / kSlotTile)
  int32_t* tile_hist;      // [ntiles, E] per-tile counts
  int32_t* tile_base;      // [ntiles, E] per-tile starting ranks
  int32_t* raw;            // [E]
  int32_t* counts;         // [E]   kept
  int32_t* offsets;        // [E+2] (E+1 used when shared_rows > 0)
  int32_t* n_dropped;      // [1]
  int shared_rows;         // T when the always-on expert follows the routed rows, else 0
  // outputs of the rank pass (any may be null)
  uint8_t* dropped;        // [n]
  int32_t* pos;            // [n]
  int32_t* row_token;      // [n + shared_rows]
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);

hipError_t launch_pack_rows(const void* x, const int32_t* row_token, const int32_t* n_rows,
                            int max_rows, int H, int elem_bytes, void* xp, hipStream_t s);

// tile map of the grouped GEMMs: tile_start[g] = sum over g' < g of ceil(rows_g' / bm) * nt,
// and (info non-null) one entry per tile t: {g, tile_start[g], offsets[g], rows of g}, so that a
// GEMM finds a tile's group with one load instead of a search over the groups
hipError_t launch_tile_map(const int32_t* offsets, int G, int bm0, int nt0, int32_t* start0,
                           int4* info0, int bm1, int nt1, int32_t* start1, int4* info1,
                           hipStream_t s);

// combine.hip
hipError_t launch_combine(const void* yp, const int32_t* pos, const float* w, const void* ys,
                          const int32_t* ys_row0, int T, int H, int k, int bf16, void* y,
                          hipStream_t s);

// gemm_bf16.hip / gemm_f32.hip: grouped GEMMs
// EPI_SWIGLU_MX8: the SwiGLU output quantised to MXFP8 (codes in c, E8M0 scales in c_mx)
enum Epilogue { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2, EPI_SWIGLU_MX8 = 3 };

struct GroupedGemm {
  // A: packed rows [*, K]; row r of group g reads A row (row_map ? row_map[r] : r)
  const void* a;
  const int32_t* row_map;
  // MXFP8 activations (with MXFP4 weights only): a holds E4M3 codes [a_rows, K] and a_mx the
  // E8M0 scales [a_rows, K/32], both row-major.  Null a_mx: a holds bf16 (or fp32) rows.
  const uint8_t* a_mx;
  int64_t a_rows;            // rows addressable in a (for range checks)
  int64_t max_rows;          // upper bound of the packed rows over all groups
  // B: per group [N_b, K] with N_b = N (or 2 panels of N for SwiGLU: b and b2)
  const void* b;             // routed group g uses b + g * b_stride
  const void* b2;            // SwiGLU second panel (W3), same strides
  int64_t b_stride;          // elements between consecutive groups' matrices
  const void* b_extra;       // the always-on group (index G_routed), or null
  const void* b2_extra;
  // FP8 E4M3 weights (one byte per element; bf16 MFMA path only): per-row fp32 scales, group g
  // of b at b_scale + g * N, of b2 at b2_scale + g * N, the extra group's at *_scale_extra.
  // Null b_scale: b and b2 hold the layer's storage type.
  const float* b_scale;
  const float* b2_scale;
  const float* b_scale_extra;
  const float* b2_scale_extra;
  // MXFP4 weights (two E2M1 codes per byte, element 2j in the low nibble; bf16 MFMA path only):
  // E8M0 scales [N, K/32] per group, b_mx + w * N * (K/32) (b2_mx for b2, *_mx_extra for the
  // extra group).  Null b_mx: no MXFP4.
  const uint8_t* b_mx;
  const uint8_t* b2_mx;
  const uint8_t* b_mx_extra;
  const uint8_t* b2_mx_extra;
  // [G_routed] or null: routed group g's weights are matrix group_slot[g] of b / b2 (an expert
  // cache's slot); null: matrix g (bf16 MFMA path only)
  const int32_t* group_slot;
  int N, K;                  // output columns, reduction length
  // output C [*, ldc]
  void* c;
  int ldc;
  uint8_t* c_mx;             // EPI_SWIGLU_MX8: E8M0 scales [*, N/32] of the MXFP8 output
  // groups
  const int32_t* offsets;    // [G+1] packed row range of each group (device) or null
  int G;                     // groups (routed + extra)
  int G_routed;
  int static_rows;           // rows of the single group when offsets == null
  const int32_t* tile_start; // [G+1] device tile map, or null with offsets == null
  const int4* tile_info;     // [tiles] per-tile entries of that map (launch_tile_map), or null
  int ksplit;                // > 1: split the reduction (fp32 output only), partial s at
  int64_t c_split_stride;    //      c + s * c_split_stride (elements)
  // Split of the last, partly filled round of tiles (each XCD's chunk): when set, a tile of
  // that round is reduced by up to 4 workgroups into fp32 partials here, which a second
  // kernel adds in a fixed order before the epilogue.  Room: 8 * kTailPieces tiles.
  float* tail_part;
};
constexpr int kTailPieces = 32;  // partial tiles per XCD the tail buffer holds

// bf16 MFMA paths
enum GemmKind { GEMM_GATE = 0, GEMM_GATE_UP = 1, GEMM_DOWN = 2 };
// tiles per group needed by the chosen configuration
void gemm_bf16_tiling(GemmKind kind, int max_rows_per_group, int N, int* bm, int* nt);
// rows of a bf16 gate tile for T tokens and E experts, split reduction or not
int gemm_gate_bm(int T, int E, bool split);
hipError_t launch_gemm_bf16(GemmKind kind, const GroupedGemm& g, int max_rows_per_group,
                            int num_cus, hipStream_t s);
// bytes of GroupedGemm::tail_part needed by launch_gemm_bf16 for this kind and group size
size_t gemm_tail_bytes(int avg_rows_per_group);

// cache.hip: the device side of an expert cache (pool slots and the expert -> slot table)
struct CacheView {
  const void *w1, *w3, *w2;  // [slots, I, H], [slots, I, H], [slots, H, I] (values or codes)
  const uint8_t *s1, *s3, *s2;  // MXFP4: the slots' E8M0 scales; else null
  bool mx;
  const int32_t* table;      // [E] expert -> slot
  int E, H, I;
};
}  // namespace moe
struct moe_expert_cache;
namespace moe {
CacheView cache_view(const moe_expert_cache* c);
// the cached layer's residency step: the experts with rows in counts[E] (device) made resident,
// decided and copied on the device on copy stream cs after the work so far on ks, which then
// waits for them
hipError_t cache_enqueue_counts(moe_expert_cache* c, const int32_t* counts, hipStream_t cs,
                                hipStream_t ks);

// quant.hip: per-row FP8 E4M3 quantisation of a [rows, K] bf16 or fp32 matrix (K % 8 == 0)
hipError_t launch_quantize_fp8(const void* w, int bf16, int64_t rows, int K, uint8_t* q,
                               float* scales, hipStream_t s);
// MXFP4 quantisation (K % 32 == 0): codes [rows, K/2], E8M0 scales [rows, K/32]
hipError_t launch_quantize_mxfp4(const void* w, int bf16, int64_t rows, int K, uint8_t* q,
                                 uint8_t* scales, hipStream_t s);
// MXFP8 quantisation of activations (K % 32 == 0): codes [rows, K] and E8M0 scales
// [rows, K/32], both row-major
hipError_t launch_quantize_mxfp8(const void* x, int bf16, int64_t rows, int K, uint8_t* q,
                                 uint8_t* scales, hipStream_t s);

// out[i] = sum_s part[s * n + i] (fixed order)
hipError_t launch_splitk_reduce(const float* part, int S, int64_t n, float* out, hipStream_t s);

// fp32 vector-FMA paths
void gemm_f32_tiling(int N, int* bm, int* nt);
hipError_t launch_gemm_f32(GemmKind kind, const GroupedGemm& g, int max_tiles, hipStream_t s);

}  // namespace moe
