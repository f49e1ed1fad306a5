// Count, capacity drop, exclusive prefix sum and stable scatter into
// expert-contiguous rows; the on-device stand-in for the dispatch step.
//
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §8: tokens are
// counted, sorted and packed by target expert before one grouped GEMM per
// expert.  "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地"
// §3.1 groups by expert id and, when bucketing decode requests, keeps request
// order inside each expert; §2.1 bounds each expert by a capacity.
//
// Slots s = t*k + j are cut into tiles of kSlotTile.  Pass 1 histograms each
// tile; pass 2 (one block) scans the tile histograms per expert (giving every
// tile its per-expert base), applies the capacity, and scans the kept counts
// into row offsets; pass 3 recomputes each tile's ranks with wavefront ballots
// (lanes with the same expert id, counted below the lane) on top of those
// bases, so a slot's rank is the number of earlier slots (= earlier tokens)
// routed to the same expert.  Ranks at or above the capacity are dropped;
// the others land at row offsets[e] + rank.  Integer work only: bit-exact.
// Batches of at most kSmallSlots slots take all three passes in one block of 16
// wavefronts (256 slots each, per-wavefront counts in LDS): the same ranks, one
// launch instead of three.
#include "common.hpp"

namespace moe {

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// A slot takes part when it exists, is not marked inactive and names an expert in [0, E);
// ids outside that range are treated as dropped rather than trusted as indices.
__device__ __forceinline__ bool slot_active(const PermuteArgs& a, int s) {
  return s < a.n && !(a.inactive && a.inactive[s]) && (unsigned)a.ids[s] < (unsigned)a.E;
}

// ---- pass 1: per-tile histogram -------------------------------------------------------------
__global__ __launch_bounds__(256) void perm_hist_kernel(PermuteArgs a) {
  __shared__ int32_t hist[kMaxExperts];
  const int tile = blockIdx.x;
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int s0 = tile * kSlotTile;
  for (int i = threadIdx.x; i < kSlotTile; i += blockDim.x) {
    const int s = s0 + i;
    if (slot_active(a, s)) atomicAdd(&hist[a.ids[s]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += blockDim.x)
    a.tile_hist[(int64_t)tile * a.E + e] = hist[e];
}

// block-wide exclusive scan of up to 2 * 1024 values (2 per thread), returns the total
template <int NT>
__device__ int block_exclusive_scan2(int* buf /*LDS [2*NT]*/, int* tmp /*LDS [NT/64]*/, int n) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  int v0 = 2 * tid < n ? buf[2 * tid] : 0;
  int v1 = 2 * tid + 1 < n ? buf[2 * tid + 1] : 0;
  int x = v0 + v1;
  // inclusive wave scan
  int inc = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < NT / kWave; ++i) {
      int c = tmp[i];
      tmp[i] = run;
      run += c;
    }
    tmp[NT / kWave] = run;
  }
  __syncthreads();
  const int excl = inc - x + tmp[wid];
  if (2 * tid < n) buf[2 * tid] = excl;
  if (2 * tid + 1 < n) buf[2 * tid + 1] = excl + v0;
  const int total = tmp[NT / kWave];
  __syncthreads();
  return total;
}

// ---- pass 2: scan (one block of 1024 threads) -----------------------------------------------
__global__ __launch_bounds__(1024) void perm_scan_kernel(PermuteArgs a) {
  __shared__ int32_t kept[2 * 1024];
  __shared__ int32_t dropped_part[1024 / kWave];
  __shared__ int32_t tmp[1024 / kWave + 1];
  const int tid = threadIdx.x;
  int my_drop = 0;
  for (int e = tid; e < a.E; e += blockDim.x) {
    // the tiles' counts of expert e, 16 loads in flight at a time (tile-major arrays: a
    // wavefront's lanes read neighbouring experts of one tile)
    const int32_t* __restrict__ hist = a.tile_hist + e;
    int32_t* __restrict__ base = a.tile_base + e;
    int run = 0;
    for (int t0 = 0; t0 < a.ntiles; t0 += 16) {
      int h[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) h[j] = t0 + j < a.ntiles ? hist[(int64_t)(t0 + j) * a.E] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (t0 + j < a.ntiles) base[(int64_t)(t0 + j) * a.E] = run;
        run += h[j];
      }
    }
    a.raw[e] = run;
    const int kp = (a.capacity >= 0 && run > a.capacity) ? a.capacity : run;
    kept[e] = kp;
    my_drop += run - kp;
  }
  __syncthreads();
  // counts out before the scan overwrites them
  for (int e = tid; e < a.E; e += blockDim.x) a.counts[e] = kept[e];
  __syncthreads();
  const int R = block_exclusive_scan2<1024>(kept, tmp, a.E);
  for (int e = tid; e < a.E; e += blockDim.x) a.offsets[e] = kept[e];
  if (tid == 0) {
    a.offsets[a.E] = R;
    if (a.shared_rows > 0) a.offsets[a.E + 1] = R + a.shared_rows;
  }
  // the always-on expert's rows follow the routed rows in token order
  if (a.shared_rows > 0 && a.row_token)
    for (int t = tid; t < a.shared_rows; t += blockDim.x) a.row_token[R + t] = t;
  // dropped total
  int v = my_drop;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  if ((tid & (kWave - 1)) == 0) dropped_part[tid / kWave] = v;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int i = 0; i < 1024 / kWave; ++i) s += dropped_part[i];
    if (a.n_dropped) *a.n_dropped = s;
  }
}

// ---- pass 3: stable ranks, drop flags and scatter ------------------------------------------
// 256 threads = 4 wavefronts; wavefront w owns slots [w*256, w*256+256) of the tile and walks
// them in 4 chunks of 64 in order.
__global__ __launch_bounds__(256) void perm_rank_kernel(PermuteArgs a) {
  __shared__ int32_t run[4][kMaxExperts];
  const int tile = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  for (int i = tid; i < 4 * a.E; i += blockDim.x) run[i / a.E][i % a.E] = 0;
  __syncthreads();
  const int s_wave = tile * kSlotTile + wid * 256;
  // per-wavefront histograms of the tile
  for (int c = 0; c < 4; ++c) {
    const int s = s_wave + c * kWave + lane;
    if (slot_active(a, s)) atomicAdd(&run[wid][a.ids[s]], 1);
  }
  __syncthreads();
  // running start of each wavefront: tile base + earlier wavefronts of this tile
  for (int e = tid; e < a.E; e += blockDim.x) {
    int b = a.tile_base[(int64_t)tile * a.E + e];
    for (int w = 0; w < 4; ++w) {
      const int h = run[w][e];
      run[w][e] = b;
      b += h;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  for (int c = 0; c < 4; ++c) {
    const int s = s_wave + c * kWave + lane;
    const bool in = s < a.n;
    const bool active = slot_active(a, s);
    const int e = active ? a.ids[s] : 0;
    // lanes of this chunk routed to the same expert
    uint64_t peers = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    if (active) {
      const int base = run[wid][e];
      const int rank = base + __popcll(peers & lanemask_lt(lane));
      const bool drop = a.capacity >= 0 && rank >= a.capacity;
      if (a.dropped) a.dropped[s] = drop ? 1 : 0;
      if (a.pos) {
        if (drop) {
          a.pos[s] = -1;
        } else {
          const int row = a.offsets[e] + rank;
          a.pos[s] = row;
          if (a.row_token) a.row_token[row] = s / a.k;
        }
      }
      // the highest lane of the group advances the running count
      if ((peers >> lane) == 1ull) run[wid][e] = base + __popcll(peers);
    } else if (in) {
      if (a.dropped) a.dropped[s] = 1;
      if (a.pos) a.pos[s] = -1;
    }
    __syncthreads();
  }
}

// ---- small batches: histogram, scan and ranks in one block ---------------------------------
// 1024 threads = 16 wavefronts; wavefront w owns slots [w*256, w*256+256) and walks them in 4
// chunks of 64 in order, as a tile's wavefronts do in perm_rank_kernel; its per-expert counts,
// then their running starts, live in LDS.
constexpr int kSmallWaves = 16;
constexpr int kSmallSlots = kSmallWaves * 256;

__global__ __launch_bounds__(1024) void perm_small_kernel(PermuteArgs a) {
  __shared__ int32_t run[kSmallWaves][kMaxExperts];
  __shared__ int32_t kept[2 * 1024];
  __shared__ int32_t dropped_part[1024 / kWave];
  __shared__ int32_t tmp[1024 / kWave + 1];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  for (int i = tid; i < kSmallWaves * a.E; i += blockDim.x) run[i / a.E][i % a.E] = 0;
  __syncthreads();
  const int s_wave = wid * 256;
  for (int c = 0; c < 4; ++c) {
    const int s = s_wave + c * kWave + lane;
    if (slot_active(a, s)) atomicAdd(&run[wid][a.ids[s]], 1);
  }
  __syncthreads();
  // per expert: the wavefronts' starting ranks (earlier wavefronts = earlier slots), the raw
  // count and the kept count
  int my_drop = 0;
  for (int e = tid; e < a.E; e += blockDim.x) {
    int b = 0;
    for (int w = 0; w < kSmallWaves; ++w) {
      const int h = run[w][e];
      run[w][e] = b;
      b += h;
    }
    a.raw[e] = b;
    const int kp = (a.capacity >= 0 && b > a.capacity) ? a.capacity : b;
    kept[e] = kp;
    a.counts[e] = kp;
    my_drop += b - kp;
  }
  __syncthreads();
  const int R = block_exclusive_scan2<1024>(kept, tmp, a.E);  // kept[e] = offsets[e] from here
  for (int e = tid; e < a.E; e += blockDim.x) a.offsets[e] = kept[e];
  if (tid == 0) {
    a.offsets[a.E] = R;
    if (a.shared_rows > 0) a.offsets[a.E + 1] = R + a.shared_rows;
  }
  if (a.shared_rows > 0 && a.row_token)
    for (int t = tid; t < a.shared_rows; t += blockDim.x) a.row_token[R + t] = t;
  int v = my_drop;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
  if (lane == 0) dropped_part[wid] = v;
  __syncthreads();
  if (tid == 0) {
    int sum = 0;
    for (int i = 0; i < 1024 / kWave; ++i) sum += dropped_part[i];
    if (a.n_dropped) *a.n_dropped = sum;
  }
  if (!a.dropped && !a.pos) return;  // counts only (the same for every thread)
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  for (int c = 0; c < 4; ++c) {
    const int s = s_wave + c * kWave + lane;
    const bool in = s < a.n;
    const bool active = slot_active(a, s);
    const int e = active ? a.ids[s] : 0;
    // lanes of this chunk routed to the same expert
    uint64_t peers = __ballot(active);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    if (active) {
      const int base = run[wid][e];
      const int rank = base + __popcll(peers & lanemask_lt(lane));
      const bool drop = a.capacity >= 0 && rank >= a.capacity;
      if (a.dropped) a.dropped[s] = drop ? 1 : 0;
      if (a.pos) {
        if (drop) {
          a.pos[s] = -1;
        } else {
          const int row = kept[e] + rank;
          a.pos[s] = row;
          if (a.row_token) a.row_token[row] = s / a.k;
        }
      }
      // the highest lane of the group advances the running count
      if ((peers >> lane) == 1ull) run[wid][e] = base + __popcll(peers);
    } else if (in) {
      if (a.dropped) a.dropped[s] = 1;
      if (a.pos) a.pos[s] = -1;
    }
    __syncthreads();
  }
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.n > 0 && a.n <= kSmallSlots) {
    perm_small_kernel<<<1, 1024, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.n <= 0) {
    // no slots: every count is zero
    perm_scan_kernel<<<1, 1024, 0, s>>>(a);
    return hipGetLastError();
  }
  perm_hist_kernel<<<a.ntiles, 256, 0, s>>>(a);
  perm_scan_kernel<<<1, 1024, 0, s>>>(a);
  if (a.dropped || a.pos) perm_rank_kernel<<<a.ntiles, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---- pack: Xp[row] = x[row_token[row]] -----------------------------------------------------
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint4* __restrict__ x,
                                                        const int32_t* __restrict__ row_token,
                                                        const int32_t* __restrict__ n_rows,
                                                        int max_rows, int row_vecs,
                                                        uint4* __restrict__ xp) {
  const int R = *n_rows;
  for (int row = blockIdx.x; row < R && row < max_rows; row += gridDim.x) {
    const int64_t src = (int64_t)row_token[row] * row_vecs;
    const int64_t dst = (int64_t)row * row_vecs;
    for (int v = threadIdx.x; v < row_vecs; v += blockDim.x) xp[dst + v] = x[src + v];
  }
}

hipError_t launch_pack_rows(const void* x, const int32_t* row_token, const int32_t* n_rows,
                            int max_rows, int H, int elem_bytes, void* xp, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const int row_vecs = H * elem_bytes / 16;  // H * elem_bytes is a multiple of 16 (checked)
  const int grid = max_rows < 4096 ? max_rows : 4096;
  pack_rows_kernel<<<grid, 256, 0, s>>>((const uint4*)x, row_token, n_rows, max_rows, row_vecs,
                                        (uint4*)xp);
  return hipGetLastError();
}

// ---- tile map of the grouped GEMMs ----------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets,
                                                        int G, int bm0, int nt0,
                                                        int32_t* __restrict__ start0,
                                                        int4* __restrict__ info0, int bm1,
                                                        int nt1, int32_t* __restrict__ start1,
                                                        int4* __restrict__ info1) {
  __shared__ int32_t buf[2 * 1024];
  __shared__ int32_t offs[2 * 1024 + 1];
  __shared__ int32_t tmp[1024 / kWave + 1];
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  for (int g = threadIdx.x; g <= G; g += blockDim.x) offs[g] = offsets[g];
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    const int bm = pass ? bm1 : bm0, nt = pass ? nt1 : nt0;
    int32_t* out = pass ? start1 : start0;
    int4* info = pass ? info1 : info0;
    if (!out) continue;
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
      const int rows = offs[g + 1] - offs[g];
      buf[g] = (rows + bm - 1) / bm * nt;
    }
    __syncthreads();
    const int total = block_exclusive_scan2<1024>(buf, tmp, G);
    for (int g = threadIdx.x; g < G; g += blockDim.x) out[g] = buf[g];
    if (threadIdx.x == 0) out[G] = total;
    if (info) {
      // tiles [buf[g], buf[g + 1]) belong to group g; wavefront w fills those of groups w,
      // w + 16, ... (a group without tiles writes nothing)
      for (int g = wid; g < G; g += blockDim.x / kWave) {
        const int t0 = buf[g], t1 = g + 1 < G ? buf[g + 1] : total;
        const int4 v = make_int4(g, t0, offs[g], offs[g + 1] - offs[g]);
        for (int t = t0 + lane; t < t1; t += kWave) info[t] = v;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_tile_map(const int32_t* offsets, int G, int bm0, int nt0, int32_t* start0,
                           int4* info0, int bm1, int nt1, int32_t* start1, int4* info1,
                           hipStream_t s) {
  tile_map_kernel<<<1, 1024, 0, s>>>(offsets, G, bm0, nt0, start0, info0, bm1, nt1, start1, info1);
  return hipGetLastError();
}

}  // namespace moe
