// C ABI of libmoe.so (declared in include/moe.h): argument checks, workspace
// carving and the launch sequence of each call.  All compute is in the kernels
// of route.hip, permute.hip, gemm_bf16.hip, gemm_f32.hip and combine.hip.
#include "../../include/moe.h"
#include "common.hpp"

#include <limits.h>
#include <math.h>

#include <atomic>
#include <vector>

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Byte layout of the workspace; one layout serves every call.
struct Layout {
  size_t tail, gate_part, logits, ids, w, tile_hist, tile_base, raw, counts, offsets, n_dropped, ts_gu, ts_dn,
      ti_gu, ti_dn, ti_cap, pos,
      dropped, row_token, xq, act, yp, yps, total;
};

// bytes of `rows` MXFP8 rows of K codes: the codes, then (256-byte aligned) their E8M0 scales
size_t mx8_bytes(size_t rows, size_t K) { return align_up(rows * K) + rows * (K / 32); }

int elem_bytes(const moe_dims_t* d) { return d->dtype == MOE_BF16 ? 2 : 4; }

// Split-K factor of the fused layer's bf16 gate: enough workgroups to fill the GPU when there
// are few (token, expert) tiles, keeping at least 4 k-steps per split.  With 128-row tiles
// (one 128-KB-LDS workgroup per CU) it aims at one workgroup per CU, since every split adds
// T x E fp32 partial sums to write and reduce.
int gate_splits(const moe_dims_t* d) {
  if (d->dtype != MOE_BF16 || d->T <= 0) return 1;
  const int bn = d->E <= 32 ? 32 : d->E <= 64 ? 64 : d->E <= 128 ? 128 : 256;
  const int bm = gemm_gate_bm(d->T, d->E, true);
  const int64_t tiles = (int64_t)ceil_div(d->T, bm) * ceil_div(d->E, bn);
  const int64_t limit = bm == 128 ? 256 : 1024;
  const int kt = d->H / 64;
  int s = 1;
  while (s < 16 && tiles * s * 2 <= limit && kt / (s * 2) >= 4) s *= 2;
  return s;
}

Layout layout(const moe_dims_t* d) {
  const size_t T = d->T, E = d->E, n = (size_t)d->T * d->k, es = elem_bytes(d);
  const size_t ntiles = (n + kSlotTile - 1) / kSlotTile;
  const bool fold = d->I_shared > 0 && d->I_shared == d->I;  // shared expert as one more group
  const size_t rows = n + (fold ? T : 0);
  const size_t imax = d->I_shared > d->I ? d->I_shared : d->I;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes ? bytes : 1);
    return at;
  };
  // partial tiles of the grouped GEMMs' split last round (sized for the larger tile shape the
  // routed experts or a separate shared expert can take)
  if (d->dtype == MOE_BF16) {
    const int64_t avg = (int64_t)d->T * d->k / d->E;
    // a shared expert of another width runs as its own group of T rows
    const bool own_shared = d->I_shared > 0 && d->I_shared != d->I;
    const int big_rows = (avg >= kBigTileRows || (own_shared && d->T >= kBigTileRows)) ? kBigTileRows : 0;
    L.tail = take(gemm_tail_bytes(big_rows));
  } else {
    L.tail = take(0);
  }
  const int gs = gate_splits(d);
  L.gate_part = take(gs > 1 ? (size_t)gs * T * E * 4 : 0);
  L.logits = take(T * E * 4);
  L.ids = take(n * 4);
  L.w = take(n * 4);
  L.tile_hist = take(E * ntiles * 4);
  L.tile_base = take(E * ntiles * 4);
  L.raw = take(E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 2) * 4);
  L.n_dropped = take(4);
  L.ts_gu = take((E + 2) * 4);
  L.ts_dn = take((E + 2) * 4);
  // per-tile entries of both tile maps: at most (rows / 32 + groups) row tiles (32-row tiles
  // give the most) times the column tiles of 128 or more columns
  {
    const size_t cols = imax > (size_t)d->H ? imax : (size_t)d->H;
    const size_t tiles = ((rows + 31) / 32 + E + 2) * ((cols + 127) / 128);
    L.ti_cap = d->dtype == MOE_BF16 ? tiles : 0;
    L.ti_gu = take(L.ti_cap * 16);
    L.ti_dn = take(L.ti_cap * 16);
  }
  L.pos = take(n * 4);
  L.dropped = take(n);
  L.row_token = take((n + T) * 4);
  // the layer's input rows in MXFP8 (layers with MXFP8 activations; bf16 layers only)
  const bool mx8 = d->dtype == MOE_BF16 && d->H % 32 == 0;
  L.xq = take(mx8 ? mx8_bytes(T, d->H) : 0);
  // the gate-up output: bf16 rows, or MXFP8 rows with their scales
  const size_t act_rows = rows > T ? rows : T;
  const size_t act_bytes = act_rows * imax * es;
  L.act = take(mx8 && mx8_bytes(act_rows, imax) > act_bytes ? mx8_bytes(act_rows, imax) : act_bytes);
  // packed expert outputs; the expert FFN call with MXFP8 activations quantises its packed input
  // rows here first
  const size_t yp_bytes = rows * (size_t)d->H * es;
  L.yp = take(mx8 && mx8_bytes(n, d->H) > yp_bytes ? mx8_bytes(n, d->H) : yp_bytes);
  L.yps = take(d->I_shared > 0 && !fold ? T * (size_t)d->H * es : 0);
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return (P*)((char*)ws + off);
}

moe_status_t check_dims(const moe_dims_t* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->H <= 0 || d->E <= 0 || d->I <= 0 || d->I_shared < 0) return MOE_ERR_INVALID_ARG;
  if (d->k < 1 || d->k > d->E) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (d->bias_mode != MOE_BIAS_SOFTMAX && d->bias_mode != MOE_BIAS_SELECT) return MOE_ERR_INVALID_ARG;
  if (d->E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->T * d->k > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_BF16) {
    if (d->H % 64 || d->I % 64 || d->I_shared % 64) return MOE_ERR_UNSUPPORTED;
    // 32-bit buffer offsets of the MFMA path
    const int64_t lim = (int64_t)1 << 31;
    const int64_t n = (int64_t)d->T * d->k + d->T;
    const int64_t imax = d->I_shared > d->I ? d->I_shared : d->I;
    if ((int64_t)d->T * d->H * 2 >= lim || n * d->H * 2 >= lim || n * imax * 2 >= lim ||
        (int64_t)imax * d->H * 2 >= lim || (int64_t)d->E * d->H * 2 >= lim)
      return MOE_ERR_UNSUPPORTED;
  } else {
    if (d->H % 4) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// compute units of the current device, queried once per device
int num_cus() {
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// record event i of the debug struct, when the caller asked for it
hipError_t mark(void* const* ev, int i, hipStream_t s) {
  if (!ev || !ev[i]) return hipSuccess;
  return hipEventRecord((hipEvent_t)ev[i], s);
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                             \
  do {                                            \
    hipError_t _e = (expr);                       \
    if (_e != hipSuccess) return MOE_ERR_HIP;     \
  } while (0)

// ---- step implementations shared by the step-wise and fused calls --------------------------

// splits > 1 needs `part` with room for splits * T * E floats
// With reduce = false a split gate stops at the partial sums in `part` (the route kernel adds
// them up).
hipError_t run_gate(const moe_dims_t* d, const void* x, const void* wg, float* logits,
                    hipStream_t s, int splits = 1, float* part = nullptr, bool reduce = true) {
  GroupedGemm p = {};
  p.a = x;
  p.a_rows = d->T;
  p.max_rows = d->T;
  p.b = wg;
  p.N = d->E;
  p.K = d->H;
  p.c = logits;
  p.ldc = d->E;
  p.G = 1;
  p.G_routed = 1;
  p.static_rows = d->T;
  if (d->dtype == MOE_BF16) {
    if (splits <= 1 || !part) return launch_gemm_bf16(GEMM_GATE, p, d->T, num_cus(), s);
    p.c = part;
    p.ksplit = splits;
    p.c_split_stride = (int64_t)d->T * d->E;
    hipError_t e = launch_gemm_bf16(GEMM_GATE, p, d->T, num_cus(), s);
    if (e != hipSuccess || !reduce) return e;
    return launch_splitk_reduce(part, splits, (int64_t)d->T * d->E, logits, s);
  }
  int bm, nt;
  gemm_f32_tiling(d->E, &bm, &nt);
  return launch_gemm_f32(GEMM_GATE, p, ceil_div(d->T, bm) * nt, s);
}

PermuteArgs permute_args(const moe_dims_t* d, const Layout& L, void* ws) {
  PermuteArgs a = {};
  a.n = d->T * d->k;
  a.k = d->k;
  a.E = d->E;
  a.T = d->T;
  a.capacity = -1;
  a.ntiles = ceil_div(a.n, kSlotTile);
  a.tile_hist = at<int32_t>(ws, L.tile_hist);
  a.tile_base = at<int32_t>(ws, L.tile_base);
  a.raw = at<int32_t>(ws, L.raw);
  a.counts = at<int32_t>(ws, L.counts);
  a.offsets = at<int32_t>(ws, L.offsets);
  a.n_dropped = at<int32_t>(ws, L.n_dropped);
  return a;
}

// weights of expert FFNs: the layer's storage type (no scales), or FP8 E4M3 codes with one
// fp32 scale per row (bf16 layers only)
struct ExpertWeights {
  const void *w1, *w3, *w2;
  const float *s1, *s3, *s2;      // FP8 E4M3: per-row scales
  const uint8_t *m1, *m3, *m2;    // MXFP4: E8M0 scales per 32 k
  bool a8 = false;                // MXFP4 weights applied to MXFP8 activations
  bool fp8() const { return s1 != nullptr; }
  bool mx() const { return m1 != nullptr; }
  int fmt() const { return fp8() ? 1 : mx() ? (a8 ? 3 : 2) : 0; }
  bool complete() const {
    const bool s = s1 && s3 && s2, no_s = !s1 && !s3 && !s2;
    const bool m = m1 && m3 && m2, no_m = !m1 && !m3 && !m2;
    return w1 && w3 && w2 && (s || no_s) && (m || no_m) && !(s && m) && (!a8 || m);
  }
};

ExpertWeights plain_weights(const void* w1, const void* w3, const void* w2) {
  return ExpertWeights{w1, w3, w2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
}
ExpertWeights fp8_weights(const void* w1, const float* s1, const void* w3, const float* s3,
                          const void* w2, const float* s2) {
  return ExpertWeights{w1, w3, w2, s1, s3, s2, nullptr, nullptr, nullptr};
}
ExpertWeights mxfp4_weights(const void* w1, const uint8_t* s1, const void* w3, const uint8_t* s3,
                            const void* w2, const uint8_t* s2) {
  return ExpertWeights{w1, w3, w2, nullptr, nullptr, nullptr, s1, s3, s2};
}
ExpertWeights w4a8_weights(const void* w1, const uint8_t* s1, const void* w3, const uint8_t* s3,
                           const void* w2, const uint8_t* s2) {
  return ExpertWeights{w1, w3, w2, nullptr, nullptr, nullptr, s1, s3, s2, true};
}

// grouped gate-up + down over G groups whose packed row ranges are offsets[0..G]; groups past
// G_routed (at most one) take the extra weights X.  With W.a8, `a` holds MXFP8 codes and a_mx
// their scales, and the activation goes through `act` in MXFP8 (codes, then the scales at
// align_up(max_rows * I)).
hipError_t run_ffn(const moe_dims_t* d, int I, const void* a, const uint8_t* a_mx,
                   const int32_t* row_map,
                   int64_t a_rows, int64_t max_rows, const int32_t* offsets, int G, int G_routed,
                   const ExpertWeights& W, const ExpertWeights* X, void* act, void* out,
                   int32_t* ts_gu, int32_t* ts_dn, int4* ti_gu, int4* ti_dn, size_t ti_cap,
                   int avg_rows,
                   float* tail, hipStream_t s,
                   void* const* ev = nullptr, const int32_t* group_slot = nullptr) {
  const bool bf16 = d->dtype == MOE_BF16;
  // groups past G_routed take the extra weights; there must be some for them, stored like W's
  if (G_routed < 0 || G_routed > G || !W.complete() || (W.fmt() && !bf16)) return hipErrorInvalidValue;
  if (G > G_routed && (!X || !X->complete() || X->fmt() != W.fmt())) return hipErrorInvalidValue;
  // MXFP4 weights on bf16 rows run on the 32-row tiles for every group size; on MXFP8 rows the
  // tiles follow the group size as for bf16
  if (W.mx() && !W.a8) avg_rows = 0;
  if (W.a8 != (a_mx != nullptr)) return hipErrorInvalidValue;
  uint8_t* act_mx = W.a8 ? (uint8_t*)act + align_up((size_t)max_rows * I) : nullptr;
  if (group_slot && !bf16) return hipErrorInvalidValue;  // slot indirection: MFMA path only
  int bm_gu, nt_gu, bm_dn, nt_dn;
  if (bf16) {
    gemm_bf16_tiling(GEMM_GATE_UP, avg_rows, I, &bm_gu, &nt_gu);
    gemm_bf16_tiling(GEMM_DOWN, avg_rows, d->H, &bm_dn, &nt_dn);
  } else {
    gemm_f32_tiling(I, &bm_gu, &nt_gu);
    gemm_f32_tiling(d->H, &bm_dn, &nt_dn);
  }
  if (!bf16) ti_gu = ti_dn = nullptr;  // the fp32 GEMMs search the map
  // per-tile entries only where the launch's tile count fits the table (else the GEMM searches)
  auto fits = [&](int bm, int nt) {
    return (size_t)((max_rows + bm - 1) / bm + G) * (size_t)nt <= ti_cap;
  };
  if (ti_gu && !fits(bm_gu, nt_gu)) ti_gu = nullptr;
  if (ti_dn && !fits(bm_dn, nt_dn)) ti_dn = nullptr;
  hipError_t e = launch_tile_map(offsets, G, bm_gu, nt_gu, ts_gu, ti_gu, bm_dn, nt_dn, ts_dn, ti_dn, s);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, MOE_EV_PERMUTE, s)) != hipSuccess) return e;

  GroupedGemm gu = {};
  gu.a = a;
  gu.a_mx = a_mx;
  gu.row_map = row_map;
  gu.a_rows = a_rows;
  gu.max_rows = max_rows;
  gu.b = W.w1;
  gu.b2 = W.w3;
  gu.b_scale = W.s1;
  gu.b2_scale = W.s3;
  gu.b_mx = W.m1;
  gu.b2_mx = W.m3;
  gu.b_stride = (int64_t)I * d->H;
  if (G > G_routed) {
    gu.b_extra = X->w1;
    gu.b2_extra = X->w3;
    gu.b_scale_extra = X->s1;
    gu.b2_scale_extra = X->s3;
    gu.b_mx_extra = X->m1;
    gu.b2_mx_extra = X->m3;
  }
  gu.N = I;
  gu.K = d->H;
  gu.c = act;
  gu.ldc = I;
  gu.c_mx = act_mx;
  gu.offsets = offsets;
  gu.G = G;
  gu.G_routed = G_routed;
  gu.tile_start = ts_gu;
  gu.tile_info = ti_gu;
  gu.group_slot = group_slot;
  gu.tail_part = bf16 ? tail : nullptr;

  GroupedGemm dn = {};
  dn.a = act;
  dn.a_mx = act_mx;
  dn.a_rows = max_rows;
  dn.max_rows = max_rows;
  dn.b = W.w2;
  dn.b_scale = W.s2;
  dn.b_mx = W.m2;
  dn.b_stride = (int64_t)d->H * I;
  if (G > G_routed) {
    dn.b_extra = X->w2;
    dn.b_scale_extra = X->s2;
    dn.b_mx_extra = X->m2;
  }
  dn.N = d->H;
  dn.K = I;
  dn.c = out;
  dn.ldc = d->H;
  dn.offsets = offsets;
  dn.G = G;
  dn.G_routed = G_routed;
  dn.tile_start = ts_dn;
  dn.tile_info = ti_dn;
  dn.group_slot = group_slot;
  dn.tail_part = bf16 ? tail : nullptr;

  const int cus = num_cus();
  const int64_t mt_gu = (ceil_div64(max_rows, bm_gu) + G) * nt_gu;
  const int64_t mt_dn = (ceil_div64(max_rows, bm_dn) + G) * nt_dn;
  e = bf16 ? launch_gemm_bf16(GEMM_GATE_UP, gu, avg_rows, cus, s)
           : launch_gemm_f32(GEMM_GATE_UP, gu, (int)mt_gu, s);
  if (e != hipSuccess) return e;
  if ((e = mark(ev, MOE_EV_GATE_UP, s)) != hipSuccess) return e;
  e = bf16 ? launch_gemm_bf16(GEMM_DOWN, dn, avg_rows, cus, s)
           : launch_gemm_f32(GEMM_DOWN, dn, (int)mt_dn, s);
  if (e != hipSuccess) return e;
  return mark(ev, MOE_EV_DOWN, s);
}

// device offsets [0, T] of a single group covering every token
__global__ void whole_range_kernel(int32_t* offsets, int T) {
  offsets[0] = 0;
  offsets[1] = T;
}

}  // namespace

extern "C" {

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_capacity(int32_t T, int32_t k, int32_t E, double factor) {
  if (E <= 0 || T < 0 || k < 0 || !(factor >= 0.0)) return -1;
  return (int32_t)floor((double)T * (double)k / (double)E * factor);
}

size_t moe_workspace_bytes(const moe_dims_t* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return layout(d).total;
}

moe_status_t moe_gate(const moe_dims_t* d, const void* x, const void* wg, float* logits,
                      void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!x || !wg || !logits) return MOE_ERR_INVALID_ARG;
  return hip_status(run_gate(d, x, wg, logits, (hipStream_t)stream));
}

moe_status_t moe_route(const moe_dims_t* d, const float* logits, const float* bias,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, uint8_t* dropped,
                       int32_t* n_dropped, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w) {
    if (d->T > 0) return MOE_ERR_INVALID_ARG;
  }
  const bool need_ws = counts || dropped || n_dropped;
  const Layout L = layout(d);
  if (need_ws && (!ws || ws_bytes < L.total)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (d->T > 0)
    MOE_TRY(launch_route(logits, bias, d->T, d->E, d->k, d->renormalize, d->bias_mode, topk_ids,
                         topk_w, s));
  if (!need_ws) return MOE_OK;
  PermuteArgs a = permute_args(d, L, ws);
  a.ids = topk_ids;
  a.capacity = d->capacity;
  if (counts) a.counts = counts;
  if (n_dropped) a.n_dropped = n_dropped;
  a.dropped = dropped;
  MOE_TRY(launch_permute(a, s));
  return MOE_OK;
}

moe_status_t moe_load_stats(const moe_dims_t* d, const int32_t* topk_ids, int32_t* raw_counts,
                            moe_load_stats_t* stats, float* bias_next, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!stats || (d->T > 0 && !topk_ids)) return MOE_ERR_INVALID_ARG;
  if (bias_next && d->capacity < 1) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // the permutation's histogram and scan give the per-expert picks (no rows are placed)
  PermuteArgs a = permute_args(d, L, ws);
  a.ids = topk_ids;
  a.capacity = d->capacity;
  if (raw_counts) a.raw = raw_counts;
  MOE_TRY(launch_permute(a, s));
  MOE_TRY(launch_load_stats(a.raw, d->E, d->capacity, stats, bias_next, s));
  return MOE_OK;
}

moe_status_t moe_permute(const moe_dims_t* d, const void* x, const int32_t* topk_ids,
                         const uint8_t* dropped, int32_t* offsets, int32_t* row_token,
                         int32_t* pos, void* x_packed, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!offsets) return MOE_ERR_INVALID_ARG;
  if (d->T > 0 && (!topk_ids || !row_token || !pos)) return MOE_ERR_INVALID_ARG;
  if (x_packed && !x) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  PermuteArgs a = permute_args(d, L, ws);
  a.ids = topk_ids;
  a.inactive = dropped;
  a.offsets = offsets;
  a.pos = pos;
  a.row_token = row_token;
  MOE_TRY(launch_permute(a, s));
  if (x_packed)
    MOE_TRY(launch_pack_rows(x, row_token, offsets + d->E, d->T * d->k, d->H, elem_bytes(d),
                             x_packed, s));
  return MOE_OK;
}

}  // extern "C"

namespace {

moe_status_t expert_ffn_impl(const moe_dims_t* d, const void* x_packed, const int32_t* offsets,
                             const ExpertWeights& W, void* y_packed, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (!offsets || !W.complete()) return MOE_ERR_INVALID_ARG;
  if (W.fmt() && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (W.mx() && (d->H % 128 || d->I % 128)) return MOE_ERR_UNSUPPORTED;
  if (d->T > 0 && (!x_packed || !y_packed)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  const int64_t n = (int64_t)d->T * d->k;
  const int avg = (int)(n / d->E);
  hipStream_t s = (hipStream_t)stream;
  const void* a = x_packed;
  const uint8_t* a_mx = nullptr;
  if (W.a8) {  // the packed rows in MXFP8, in the packed-output area (unused by this call)
    uint8_t* xq = at<uint8_t>(ws, L.yp);
    a_mx = xq + align_up((size_t)n * d->H);
    MOE_TRY(launch_quantize_mxfp8(x_packed, 1, n, d->H, xq, (uint8_t*)a_mx, s));
    a = xq;
  }
  MOE_TRY(run_ffn(d, d->I, a, a_mx, nullptr, n, n, offsets, d->E, d->E, W, nullptr,
                  at<void>(ws, L.act), y_packed, at<int32_t>(ws, L.ts_gu),
                  at<int32_t>(ws, L.ts_dn), at<int4>(ws, L.ti_gu), at<int4>(ws, L.ti_dn), L.ti_cap, avg, at<float>(ws, L.tail), s));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_expert_ffn(const moe_dims_t* d, const void* x_packed, const int32_t* offsets,
                            const void* w1, const void* w3, const void* w2, void* y_packed,
                            void* ws, size_t ws_bytes, void* stream) {
  return expert_ffn_impl(
      d, x_packed, offsets,
      plain_weights(w1, w3, w2), y_packed,
      ws, ws_bytes, stream);
}

moe_status_t moe_expert_ffn_fp8(const moe_dims_t* d, const void* x_packed,
                                const int32_t* offsets, const uint8_t* w1q, const float* w1s,
                                const uint8_t* w3q, const float* w3s, const uint8_t* w2q,
                                const float* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!w1s || !w3s || !w2s) return MOE_ERR_INVALID_ARG;
  return expert_ffn_impl(d, x_packed, offsets,
                         fp8_weights(w1q, w1s, w3q, w3s, w2q, w2s),
                         y_packed, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_mxfp4(int64_t rows, int32_t K, int32_t dtype, const void* w,
                                uint8_t* q, uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || (dtype != MOE_BF16 && dtype != MOE_F32)) return MOE_ERR_INVALID_ARG;
  if (K % 128 || rows % 32) return MOE_ERR_UNSUPPORTED;  // the blocked scale layout
  if (rows == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_quantize_mxfp4(w, dtype == MOE_BF16, rows, K, q, scales, (hipStream_t)stream));
  return MOE_OK;
}

moe_status_t moe_expert_ffn_mxfp4(const moe_dims_t* d, const void* x_packed,
                                  const int32_t* offsets, const uint8_t* w1q, const uint8_t* w1s,
                                  const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                  const uint8_t* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!w1s || !w3s || !w2s) return MOE_ERR_INVALID_ARG;
  return expert_ffn_impl(d, x_packed, offsets,
                         mxfp4_weights(w1q, w1s, w3q, w3s, w2q, w2s),
                         y_packed, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_mxfp8(int64_t rows, int32_t K, int32_t dtype, const void* x,
                                uint8_t* q, uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || (dtype != MOE_BF16 && dtype != MOE_F32)) return MOE_ERR_INVALID_ARG;
  if (K % 32) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_quantize_mxfp8(x, dtype == MOE_BF16, rows, K, q, scales, (hipStream_t)stream));
  return MOE_OK;
}

moe_status_t moe_expert_ffn_w4a8(const moe_dims_t* d, const void* x_packed,
                                 const int32_t* offsets, const uint8_t* w1q, const uint8_t* w1s,
                                 const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                 const uint8_t* w2s, void* y_packed, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!w1s || !w3s || !w2s) return MOE_ERR_INVALID_ARG;
  return expert_ffn_impl(d, x_packed, offsets, w4a8_weights(w1q, w1s, w3q, w3s, w2q, w2s),
                         y_packed, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_fp8(int64_t rows, int32_t K, int32_t dtype, const void* w, uint8_t* q,
                              float* scales, void* stream) {
  if (rows < 0 || K <= 0 || (dtype != MOE_BF16 && dtype != MOE_F32)) return MOE_ERR_INVALID_ARG;
  if (K % 8) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!w || !q || !scales) return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_quantize_fp8(w, dtype == MOE_BF16, rows, K, q, scales, (hipStream_t)stream));
  return MOE_OK;
}

moe_status_t moe_combine(const moe_dims_t* d, const void* y_packed, const int32_t* pos,
                         const float* topk_w, const void* y_shared, void* y, void* stream) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (!y_packed || !pos || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_combine(y_packed, pos, topk_w, y_shared, nullptr, d->T, d->H, d->k,
                         d->dtype == MOE_BF16, y, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"

namespace {

// an expert cache the routed weights come from (moe_layer_forward_cached)
struct CacheUse {
  moe_expert_cache_t* cache;
  hipStream_t copy_stream;
  moe_cache_step_t* info;
  bool a8;  // MXFP4 experts on MXFP8 activations: the cache must hold MXFP4 codes and scales
};

moe_status_t layer_forward_impl(const moe_dims_t* d, const void* x, const void* wg,
                                const float* bias, const ExpertWeights& W_in,
                                const ExpertWeights& SW, void* y, const moe_debug_out_t* dbg,
                                void* ws, size_t ws_bytes, void* stream,
                                const CacheUse* cu = nullptr) {
  moe_status_t st = check_dims(d);
  if (st != MOE_OK) return st;
  ExpertWeights W = W_in;
  const int32_t* group_slot = nullptr;
  if (cu) {
    if (d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const CacheView v = cache_view(cu->cache);
    if (v.E != d->E || v.H != d->H || v.I != d->I) return MOE_ERR_INVALID_ARG;
    if (v.mx != cu->a8) return MOE_ERR_INVALID_ARG;  // the cache's format is the entry point's
    W = v.mx ? w4a8_weights(v.w1, v.s1, v.w3, v.s3, v.w2, v.s2) : plain_weights(v.w1, v.w3, v.w2);
    group_slot = v.table;
  }
  if (!x || !wg || !W.complete() || !y) {
    if (d->T > 0) return MOE_ERR_INVALID_ARG;
  }
  if (W.fmt() && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (W.mx() && (d->H % 128 || d->I % 128 || d->I_shared % 128)) return MOE_ERR_UNSUPPORTED;
  if (d->I_shared > 0 && (!SW.complete() || SW.fmt() != W.fmt())) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  const int T = d->T, E = d->E, k = d->k, n = T * k;
  const bool shared = d->I_shared > 0;
  const bool fold = shared && d->I_shared == d->I;
  float* logits = dbg && dbg->logits ? dbg->logits : at<float>(ws, L.logits);
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* w = at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* pos = at<int32_t>(ws, L.pos);
  int32_t* row_token = at<int32_t>(ws, L.row_token);

  void* const* ev = dbg ? dbg->events : nullptr;
  // 1. gate  2. softmax / top-k / renormalise
  MOE_TRY(mark(ev, MOE_EV_START, s));
  // a split gate leaves partial sums; the route kernel adds them (in the reduction's order) and
  // writes the logits
  const int gs = gate_splits(d);
  float* gpart = at<float>(ws, L.gate_part);
  const bool fused_sum = d->dtype == MOE_BF16 && gs > 1;
  MOE_TRY(run_gate(d, x, wg, logits, s, gs, gpart, !fused_sum));
  MOE_TRY(mark(ev, MOE_EV_GATE, s));
  MOE_TRY(launch_route(logits, bias, T, E, k, d->renormalize, d->bias_mode, ids, w, s,
                       fused_sum ? gpart : nullptr, gs, fused_sum ? logits : nullptr));
  MOE_TRY(mark(ev, MOE_EV_ROUTE, s));
  // 3. count, capacity, scan, stable scatter (rows of the folded shared expert appended)
  PermuteArgs a = permute_args(d, L, ws);
  a.ids = ids;
  a.capacity = d->capacity;
  a.shared_rows = fold ? T : 0;
  a.dropped = at<uint8_t>(ws, L.dropped);
  a.pos = pos;
  a.row_token = row_token;
  MOE_TRY(launch_permute(a, s));
  if (cu) {
    // the experts with kept rows must be resident: the cache decides on the device from the
    // per-expert counts and copies the missing experts in on the copy stream, and this stream
    // waits for them (no host round trip)
    MOE_TRY(cache_enqueue_counts(cu->cache, at<int32_t>(ws, L.counts), cu->copy_stream, s));
  }
  // 4-5. grouped gate-up (rows gathered straight from x) and down
  const int G = E + (fold ? 1 : 0);
  const int64_t max_rows = (int64_t)n + (fold ? T : 0);
  const int avg = n / E;
  void* yp = at<void>(ws, L.yp);
  // MXFP8 activations: the token rows are quantised once, and the expert GEMMs gather them
  const void* xa = x;
  const uint8_t* xa_mx = nullptr;
  if (W.a8) {
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    xa_mx = xq + align_up((size_t)T * d->H);
    MOE_TRY(launch_quantize_mxfp8(x, 1, T, d->H, xq, (uint8_t*)xa_mx, s));
    xa = xq;
  }
  MOE_TRY(run_ffn(d, d->I, xa, xa_mx, row_token, T, max_rows, offsets, G, E, W, fold ? &SW : nullptr,
                  at<void>(ws, L.act), yp, at<int32_t>(ws, L.ts_gu), at<int32_t>(ws, L.ts_dn),
                  at<int4>(ws, L.ti_gu), at<int4>(ws, L.ti_dn), L.ti_cap, avg,
                  at<float>(ws, L.tail), s, ev, group_slot));
  const void* ys = nullptr;
  const int32_t* ys_row0 = nullptr;
  if (fold) {
    ys = yp;
    ys_row0 = offsets + E;  // the shared rows start after the R routed rows
  } else if (shared) {
    // a shared expert of another inner size runs as its own single-group FFN over x; the
    // tile maps, the activation buffer and `raw` (free once the permute has run) are reused
    // in stream order
    int32_t* off2 = at<int32_t>(ws, L.raw);  // two ints: [0, T]
    whole_range_kernel<<<1, 1, 0, s>>>(off2, T);
    MOE_TRY(hipGetLastError());
    MOE_TRY(run_ffn(d, d->I_shared, xa, xa_mx, nullptr, T, T, off2, 1, 1, SW, nullptr,
                    at<void>(ws, L.act), at<void>(ws, L.yps), at<int32_t>(ws, L.ts_gu),
                    at<int32_t>(ws, L.ts_dn), at<int4>(ws, L.ti_gu), at<int4>(ws, L.ti_dn), L.ti_cap, T, at<float>(ws, L.tail), s));
    ys = at<void>(ws, L.yps);
  }
  // 6. weighted combine back into token order
  MOE_TRY(launch_combine(yp, pos, w, ys, ys_row0, T, d->H, k, d->dtype == MOE_BF16, y, s));
  MOE_TRY(mark(ev, MOE_EV_END, s));

  if (dbg) {
    if (dbg->topk_ids)
      MOE_TRY(hipMemcpyAsync(dbg->topk_ids, ids, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->topk_w)
      MOE_TRY(hipMemcpyAsync(dbg->topk_w, w, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->counts)
      MOE_TRY(hipMemcpyAsync(dbg->counts, at<int32_t>(ws, L.counts), (size_t)E * 4,
                             hipMemcpyDeviceToDevice, s));
    if (dbg->offsets)
      MOE_TRY(hipMemcpyAsync(dbg->offsets, offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice,
                             s));
    if (dbg->pos) MOE_TRY(hipMemcpyAsync(dbg->pos, pos, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    if (dbg->n_dropped)
      MOE_TRY(hipMemcpyAsync(dbg->n_dropped, at<int32_t>(ws, L.n_dropped), 4,
                             hipMemcpyDeviceToDevice, s));
  }
  // the cache's residency step, when the caller asked for it: waits for the step itself
  if (cu && cu->info) return moe_cache_last_step(cu->cache, cu->info);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_layer_forward(const moe_dims_t* d, const void* x, const void* wg,
                               const float* bias, const void* w1, const void* w3, const void* w2,
                               const void* ws1, const void* ws3, const void* ws2, void* y,
                               const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                               void* stream) {
  return layer_forward_impl(d, x, wg, bias, plain_weights(w1, w3, w2),
                            plain_weights(ws1, ws3, ws2), y, dbg, ws,
                            ws_bytes, stream);
}

moe_status_t moe_layer_forward_cached(const moe_dims_t* d, const void* x, const void* wg,
                                      const float* bias, moe_expert_cache_t* cache,
                                      const void* ws1, const void* ws3, const void* ws2, void* y,
                                      const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                      void* stream, void* copy_stream, moe_cache_step_t* info) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  if (info) *info = moe_cache_step_t{};
  const CacheUse cu{cache, (hipStream_t)copy_stream, info, false};
  return layer_forward_impl(d, x, wg, bias, ExpertWeights{},
                            plain_weights(ws1, ws3, ws2), y, dbg, ws,
                            ws_bytes, stream, &cu);
}

moe_status_t moe_layer_forward_cached_w4a8(const moe_dims_t* d, const void* x, const void* wg,
                                           const float* bias, moe_expert_cache_t* cache,
                                           const uint8_t* ws1q, const uint8_t* ws1s,
                                           const uint8_t* ws3q, const uint8_t* ws3s,
                                           const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                           const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                           void* stream, void* copy_stream,
                                           moe_cache_step_t* info) {
  if (!cache) return MOE_ERR_INVALID_ARG;
  if (info) *info = moe_cache_step_t{};
  if (d && d->I_shared > 0 && (!ws1s || !ws3s || !ws2s)) return MOE_ERR_INVALID_ARG;
  const CacheUse cu{cache, (hipStream_t)copy_stream, info, true};
  return layer_forward_impl(d, x, wg, bias, ExpertWeights{},
                            w4a8_weights(ws1q, ws1s, ws3q, ws3s, ws2q, ws2s), y, dbg, ws,
                            ws_bytes, stream, &cu);
}

moe_status_t moe_layer_forward_mxfp4(const moe_dims_t* d, const void* x, const void* wg,
                                     const float* bias, const uint8_t* w1q, const uint8_t* w1s,
                                     const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                     const uint8_t* w2s, const uint8_t* ws1q, const uint8_t* ws1s,
                                     const uint8_t* ws3q, const uint8_t* ws3s,
                                     const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                     const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (d && d->T > 0 && (!w1s || !w3s || !w2s)) return MOE_ERR_INVALID_ARG;
  if (d && d->I_shared > 0 && (!ws1s || !ws3s || !ws2s)) return MOE_ERR_INVALID_ARG;
  return layer_forward_impl(
      d, x, wg, bias, mxfp4_weights(w1q, w1s, w3q, w3s, w2q, w2s),
      mxfp4_weights(ws1q, ws1s, ws3q, ws3s, ws2q, ws2s), y, dbg, ws,
      ws_bytes, stream);
}

moe_status_t moe_layer_forward_w4a8(const moe_dims_t* d, const void* x, const void* wg,
                                    const float* bias, const uint8_t* w1q, const uint8_t* w1s,
                                    const uint8_t* w3q, const uint8_t* w3s, const uint8_t* w2q,
                                    const uint8_t* w2s, const uint8_t* ws1q, const uint8_t* ws1s,
                                    const uint8_t* ws3q, const uint8_t* ws3s,
                                    const uint8_t* ws2q, const uint8_t* ws2s, void* y,
                                    const moe_debug_out_t* dbg, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (d && d->T > 0 && (!w1s || !w3s || !w2s)) return MOE_ERR_INVALID_ARG;
  if (d && d->I_shared > 0 && (!ws1s || !ws3s || !ws2s)) return MOE_ERR_INVALID_ARG;
  return layer_forward_impl(
      d, x, wg, bias, w4a8_weights(w1q, w1s, w3q, w3s, w2q, w2s),
      w4a8_weights(ws1q, ws1s, ws3q, ws3s, ws2q, ws2s), y, dbg, ws,
      ws_bytes, stream);
}

moe_status_t moe_layer_forward_fp8(const moe_dims_t* d, const void* x, const void* wg,
                                   const float* bias, const uint8_t* w1q, const float* w1s,
                                   const uint8_t* w3q, const float* w3s, const uint8_t* w2q,
                                   const float* w2s, const uint8_t* ws1q, const float* ws1s,
                                   const uint8_t* ws3q, const float* ws3s, const uint8_t* ws2q,
                                   const float* ws2s, void* y, const moe_debug_out_t* dbg,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (d && d->T > 0 && (!w1s || !w3s || !w2s)) return MOE_ERR_INVALID_ARG;
  if (d && d->I_shared > 0 && (!ws1s || !ws3s || !ws2s)) return MOE_ERR_INVALID_ARG;
  return layer_forward_impl(
      d, x, wg, bias, fp8_weights(w1q, w1s, w3q, w3s, w2q, w2s),
      fp8_weights(ws1q, ws1s, ws3q, ws3s, ws2q, ws2s), y, dbg, ws,
      ws_bytes, stream);
}

}  // extern "C"
