// Routing load statistics and the next auxiliary-loss-free balancing bias.
//
// "MoE 推理中的 Expert Parallel、KV Cache 与大规模专家并行架构解析" §11 lists the
// routing metrics to watch: the variance of expert load, the drop rate and how
// hot the hottest expert runs; "MoE Expert Parallelism 实战：稀疏大模型推理的通信与
// 负载均衡治理" asks for every expert's token count and the skew of their
// distribution.  "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程
// 落地" §2.1 sets each expert's balancing bias from its overflow over the
// capacity, clamped to [-1, 1]; its comment says an overloaded expert gets a
// negative bias (fewer tokens follow), which fixes the sign:
// b[e] = clamp((C - picks[e]) / C, -1, 1).
//
// One block of 1024 threads, thread e owning expert e.  Integer results are
// exact; the sums of squares are fp64 in a fixed order (wavefront butterfly,
// then the 16 wavefront partials in order), rounded once to fp32.
#include "../../include/moe.h"
#include "common.hpp"

namespace moe {

template <typename V, typename F>
__device__ __forceinline__ V wave_reduce(V v, F op) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = op(v, __shfl_xor(v, off, kWave));
  return v;
}

__global__ __launch_bounds__(1024) void load_stats_kernel(const int32_t* __restrict__ raw, int E,
                                                          int capacity,
                                                          moe_load_stats_t* __restrict__ st,
                                                          float* __restrict__ bias_next) {
  constexpr int NW = 1024 / kWave;
  __shared__ int64_t s_pick[NW], s_drop[NW], s_idle[NW];
  __shared__ uint64_t s_max[NW];
  __shared__ int32_t s_min[NW];
  __shared__ double s_sq[NW];
  __shared__ double s_mean;
  __shared__ int32_t s_maxcount;
  const int e = threadIdx.x, lane = e & (kWave - 1), wid = e / kWave;
  const bool live = e < E;
  const int r = live ? raw[e] : 0;

  auto add64 = [](int64_t a, int64_t b) { return a + b; };
  const int64_t pick = wave_reduce<int64_t>(r, add64);
  const int64_t drop = wave_reduce<int64_t>(live && capacity >= 0 && r > capacity ? r - capacity : 0, add64);
  const int64_t idle = wave_reduce<int64_t>(live && r == 0 ? 1 : 0, add64);
  // most picks, lowest id among equals: the largest (count, ~id) word
  const uint64_t mkey = live ? ((uint64_t)(uint32_t)r << 32) | (uint32_t)(~(uint32_t)e) : 0;
  const uint64_t mx = wave_reduce<uint64_t>(mkey, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  const int32_t mn = wave_reduce<int32_t>(live ? r : INT32_MAX, [](int32_t a, int32_t b) { return a < b ? a : b; });
  if (lane == 0) {
    s_pick[wid] = pick;
    s_drop[wid] = drop;
    s_idle[wid] = idle;
    s_max[wid] = mx;
    s_min[wid] = mn;
  }
  __syncthreads();
  if (e == 0) {
    int64_t p = 0, d = 0, z = 0;
    uint64_t m = 0;
    int32_t lo = INT32_MAX;
    for (int w = 0; w < NW; ++w) {
      p += s_pick[w];
      d += s_drop[w];
      z += s_idle[w];
      m = s_max[w] > m ? s_max[w] : m;
      lo = s_min[w] < lo ? s_min[w] : lo;
    }
    s_mean = (double)p / (double)E;
    s_maxcount = (int32_t)(m >> 32);
    st->picks = (int32_t)p;
    st->dropped = (int32_t)d;
    st->max_count = (int32_t)(m >> 32);
    st->hottest = (int32_t)(~(uint32_t)m);
    st->min_count = lo;
    st->idle = (int32_t)z;
    st->drop_rate = p > 0 ? (float)((double)d / (double)p) : 0.f;
  }
  __syncthreads();
  const double mean = s_mean;
  const double dev = live ? (double)r - mean : 0.0;
  const double sq = wave_reduce<double>(dev * dev, [](double a, double b) { return a + b; });
  if (lane == 0) s_sq[wid] = sq;
  if (bias_next && live) {
    double b = ((double)capacity - (double)r) / (double)capacity;
    b = b < -1.0 ? -1.0 : (b > 1.0 ? 1.0 : b);
    bias_next[e] = (float)b;
  }
  __syncthreads();
  if (e == 0) {
    double ss = 0.0;
    for (int w = 0; w < NW; ++w) ss += s_sq[w];
    const double sd = sqrt(ss / (double)E);
    st->mean = (float)mean;
    st->stddev = (float)sd;
    st->cv = mean > 0.0 ? (float)(sd / mean) : 0.f;
    st->max_over_mean = mean > 0.0 ? (float)((double)s_maxcount / mean) : 0.f;
  }
}

hipError_t launch_load_stats(const int32_t* raw, int E, int capacity, void* stats,
                             float* bias_next, hipStream_t s) {
  load_stats_kernel<<<1, 1024, 0, s>>>(raw, E, capacity, (moe_load_stats_t*)stats, bias_next);
  return hipGetLastError();
}

}  // namespace moe
