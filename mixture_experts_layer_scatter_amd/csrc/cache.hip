// Expert cache: the routed experts' weights resident in HBM up to a number of slots.
//
// "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地" §3.2 keeps a
// subset of the experts in HBM and loads the others from host memory before a
// batch needs them, evicting the least recently used, with the loads running
// asynchronously to the host so that they can overlap compute.  Here the pool
// (W1, W3, W2 per slot, the residency state and the device expert -> slot
// table) is caller-allocated device memory, holding the experts in the layer's
// bf16 or as MXFP4 codes and scales (§5.2 of the same page serves with the
// expert cache and 4-bit experts together, so a slot then costs a quarter of
// the bytes).  The grouped GEMMs read expert e's weights from slot table[e]
// (GroupedGemm::group_slot).
//
// Everything runs on the device, in stream order: a one-workgroup kernel
// decides a batch's residency from the per-expert row counts the permutation
// left on the device (or from a host list, moe_cache_load) and writes the list
// of experts to copy; a copy kernel then reads those experts straight from the
// pinned host arrays over PCIe into their slots.  No host round trip sits in
// the middle of a layer.
//
// Residency policy: recency = the last batch that requested an expert (ties:
// lower id); a batch's own experts are never evicted for it; free slots are
// taken lowest first; missing experts load in ascending id order; a batch that
// needs more experts than there are slots changes nothing.
#include "../../include/moe.h"
#include "common.hpp"

#include <algorithm>
#include <new>
#include <vector>

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

constexpr int kPlanThreads = 1024;      // one thread per expert and per slot
constexpr int kMaxSlots = kPlanThreads;
constexpr int kCopyBlocks = 256;  // the copy kernel's grid (PCIe-bound from 256 workgroups up)

// words of the residency state's statistics (the last planned batch)
enum { ST_STEP = 0, ST_STATUS, ST_REQUESTED, ST_HITS, ST_LOADS, ST_EVICTIONS, ST_WORDS = 8 };

// Pool: W1, W3, W2 slots (bf16 values or MXFP4 codes), then (MXFP4) their scale slots, then
// the table and the residency state.  An MXFP4 expert's codes and scales are each one
// contiguous block, as moe_quantize_mxfp4 writes them for [E * I, H] and [E * H, I].
struct PoolLayout {
  size_t part[6];  // W1, W3, W2 (values or codes), then the three scale regions
  size_t table, owner, last_use, copy_e, copy_s, stats, total;
  size_t part_bytes[6];  // bytes of one expert in each part (0: unused)
};

bool cache_dims_ok(const moe_dims_t* d, bool mx) {
  if (!d || d->H <= 0 || d->E <= 0 || d->E > moe::kMaxExperts || d->I <= 0 ||
      d->dtype != MOE_BF16)
    return false;
  return mx ? d->H % 128 == 0 && d->I % 128 == 0 : d->H % 64 == 0 && d->I % 64 == 0;
}

PoolLayout pool_layout(const moe_dims_t* d, int slots, bool mx) {
  PoolLayout L;
  const size_t n = (size_t)d->I * d->H;
  for (int i = 0; i < 3; ++i) {
    L.part_bytes[i] = mx ? n / 2 : n * 2;
    L.part_bytes[3 + i] = mx ? n / 32 : 0;
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  for (int i = 0; i < 6; ++i) L.part[i] = take((size_t)slots * L.part_bytes[i]);
  L.table = take((size_t)d->E * 4);
  L.owner = take((size_t)slots * 4);
  L.last_use = take((size_t)d->E * 4);
  L.copy_e = take((size_t)slots * 4);
  L.copy_s = take((size_t)slots * 4);
  L.stats = take(ST_WORDS * 4);
  L.total = o;
  return L;
}

struct DevState {
  int32_t *table, *owner, *last_use, *copy_e, *copy_s, *stats;
  int E, slots;
};

// A batch's request: experts named by a host list (n >= 0), else those with kept rows in
// counts[E]
struct PlanRequest {
  int n;
  uint16_t ids[moe::kMaxExperts];
};

__global__ __launch_bounds__(kPlanThreads) void cache_init_kernel(DevState st) {
  const int t = threadIdx.x;
  if (t < st.E) {
    st.table[t] = -1;
    st.last_use[t] = -1;
  }
  if (t < st.slots) st.owner[t] = -1;
  if (t < ST_WORDS) st.stats[t] = 0;
}

// exclusive rank of this thread's flag among the block's set flags, and their total
__device__ __forceinline__ int flag_rank(bool f, int* wave_cnt, int& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t b = __ballot(f);
  const int in_wave = __popcll(b & ((1ull << lane) - 1));
  if (lane == 0) wave_cnt[w] = __popcll(b);
  __syncthreads();
  int before = 0;
  total = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    if (i < w) before += wave_cnt[i];
    total += wave_cnt[i];
  }
  __syncthreads();  // wave_cnt is reused by the next call
  return before + in_wave;
}

// One batch's residency decision (thread e: expert e; thread s: slot s), then the state update
// and the copy list.  Deterministic: every choice is a rank over fixed keys.
__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(DevState st,
                                                                  const int32_t* counts,
                                                                  PlanRequest req) {
  __shared__ int s_need[moe::kMaxExperts], s_table[moe::kMaxExperts], s_last[moe::kMaxExperts];
  __shared__ int s_cand[moe::kMaxExperts];
  __shared__ int s_miss_list[moe::kMaxExperts], s_free_list[kMaxSlots], s_victim[moe::kMaxExperts];
  __shared__ int wave_cnt[kPlanThreads / 64];
  const int t = threadIdx.x, E = st.E;
  if (t < E) {
    s_table[t] = st.table[t];
    s_last[t] = st.last_use[t];
    s_need[t] = req.n < 0 ? (counts[t] > 0) : 0;
  }
  __syncthreads();
  for (int i = t; i < req.n; i += kPlanThreads) s_need[req.ids[i]] = 1;  // same value if repeated
  __syncthreads();
  const bool need = t < E && s_need[t];
  const bool hit = need && s_table[t] >= 0;
  const bool miss = need && s_table[t] < 0;
  const bool cand = t < E && !s_need[t] && s_table[t] >= 0;  // may be evicted for this batch
  const bool fre = t < st.slots && st.owner[t] < 0;
  if (t < E) s_cand[t] = cand;
  int n_need, n_hit, n_miss, n_free, n_cand;
  (void)flag_rank(need, wave_cnt, n_need);
  (void)flag_rank(hit, wave_cnt, n_hit);
  const int rank_miss = flag_rank(miss, wave_cnt, n_miss);
  const int rank_free = flag_rank(fre, wave_cnt, n_free);
  (void)flag_rank(cand, wave_cnt, n_cand);
  const int step = st.stats[ST_STEP] + 1;
  if (n_miss > n_free + n_cand) {  // more experts than slots: nothing changes
    if (t == 0) {
      st.stats[ST_STATUS] = 1;
      st.stats[ST_REQUESTED] = n_need;
      st.stats[ST_HITS] = 0;
      st.stats[ST_LOADS] = 0;
      st.stats[ST_EVICTIONS] = 0;
    }
    return;
  }
  const int n_evict = n_miss > n_free ? n_miss - n_free : 0;
  // eviction order: least recent first, ties to the lower id
  if (cand) {
    int rank = 0;
    const int lt = s_last[t];
    for (int u = 0; u < E; ++u)
      rank += s_cand[u] && (s_last[u] < lt || (s_last[u] == lt && u < t));
    if (rank < n_evict) s_victim[rank] = t;
  }
  if (miss) s_miss_list[rank_miss] = t;
  if (fre) s_free_list[rank_free] = t;
  __syncthreads();
  // the i-th missing expert (ascending id) takes the i-th free slot, then the slot of the
  // (i - free)-th eviction; every index written below is distinct
  if (t < n_miss) {
    const int e = s_miss_list[t];
    int s;
    if (t < n_free) {
      s = s_free_list[t];
    } else {
      const int v = s_victim[t - n_free];
      s = s_table[v];
      st.table[v] = -1;
    }
    st.table[e] = s;
    st.owner[s] = e;
    st.copy_e[t] = e;
    st.copy_s[t] = s;
  }
  if (need) st.last_use[t] = step;
  if (t == 0) {
    st.stats[ST_STEP] = step;
    st.stats[ST_STATUS] = 0;
    st.stats[ST_REQUESTED] = n_need;
    st.stats[ST_HITS] = n_hit;
    st.stats[ST_LOADS] = n_miss;
    st.stats[ST_EVICTIONS] = n_evict;
  }
}

// the parts of one expert to copy: host (device-visible) source, pool destination, bytes
struct CopySpec {
  const char* src[6];
  char* dst[6];
  int64_t bytes[6];
  int64_t chunk_start[7];  // 16-byte chunks of one expert before each part
};

// Copies the planned experts from pinned host memory (read over PCIe) into their slots; each
// thread moves four 16-byte chunks at a time to keep enough reads in flight.
__global__ __launch_bounds__(256) void cache_copy_kernel(const int32_t* stats, const int32_t* copy_e,
                                                        const int32_t* copy_s, CopySpec c) {
  const int n = stats[ST_STATUS] ? 0 : stats[ST_LOADS];
  const int64_t per = c.chunk_start[6], total = per * n;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  auto addr = [&](int64_t i, const uint4*& src, uint4*& dst) {
    const int item = (int)(i / per);
    const int64_t r = i - (int64_t)item * per;
    int part = 0;
    while (part < 5 && r >= c.chunk_start[part + 1]) ++part;
    const int64_t off = (r - c.chunk_start[part]) * 16;
    src = (const uint4*)(c.src[part] + (int64_t)copy_e[item] * c.bytes[part] + off);
    dst = (uint4*)(c.dst[part] + (int64_t)copy_s[item] * c.bytes[part] + off);
  };
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < total; i += 4 * stride) {
    const uint4 *s0, *s1, *s2, *s3;
    uint4 *d0, *d1, *d2, *d3;
    addr(i, s0, d0);
    addr(i + stride, s1, d1);
    addr(i + 2 * stride, s2, d2);
    addr(i + 3 * stride, s3, d3);
    const uint4 a = *s0, b = *s1, e = *s2, f = *s3;
    *d0 = a;
    *d1 = b;
    *d2 = e;
    *d3 = f;
  }
  for (; i < total; i += stride) {
    const uint4* s0;
    uint4* d0;
    addr(i, s0, d0);
    *d0 = *s0;
  }
}

}  // namespace

struct moe_expert_cache {
  int E, H, I, slots;
  bool mx;  // MXFP4 codes and scales (else bf16 values)
  DevState st;
  CopySpec copy;
  int64_t expert_bytes;  // bytes of one expert copied in
  char* pool;
  size_t part_off[6];
  bool state_ready;      // the device state has been initialised
  bool ev_valid;         // ev_state covers this cache's last plan and copy
  hipEvent_t ev_state, ev_compute;
};

namespace moe {

CacheView cache_view(const moe_expert_cache* c) {
  CacheView v;
  v.w1 = c->pool + c->part_off[0];
  v.w3 = c->pool + c->part_off[1];
  v.w2 = c->pool + c->part_off[2];
  v.s1 = c->mx ? (const uint8_t*)(c->pool + c->part_off[3]) : nullptr;
  v.s3 = c->mx ? (const uint8_t*)(c->pool + c->part_off[4]) : nullptr;
  v.s2 = c->mx ? (const uint8_t*)(c->pool + c->part_off[5]) : nullptr;
  v.mx = c->mx;
  v.table = c->st.table;
  v.E = c->E;
  v.H = c->H;
  v.I = c->I;
  return v;
}

}  // namespace moe

namespace {

// Plan a batch (counts on the device, or a host list) and copy its missing experts, on
// `copy_stream` after the work enqueued so far on `stream` (which may still read slots about to
// be refilled) and after this cache's earlier plans; `stream`'s later work waits for both.
hipError_t enqueue_residency(moe_expert_cache* c, const int32_t* counts, const PlanRequest* req,
                             hipStream_t cs, hipStream_t ks) {
  if (cs != ks) {
    hipError_t e = hipEventRecord(c->ev_compute, ks);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, c->ev_compute, 0);
    if (e != hipSuccess) return e;
  }
  if (c->ev_valid) {
    const hipError_t e = hipStreamWaitEvent(cs, c->ev_state, 0);
    if (e != hipSuccess) return e;
  }
  if (!c->state_ready) {
    cache_init_kernel<<<1, kPlanThreads, 0, cs>>>(c->st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    c->state_ready = true;
  }
  PlanRequest r;
  r.n = -1;
  if (req) r = *req;
  cache_plan_kernel<<<1, kPlanThreads, 0, cs>>>(c->st, counts, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  cache_copy_kernel<<<kCopyBlocks, 256, 0, cs>>>(c->st.stats, c->st.copy_e, c->st.copy_s, c->copy);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipEventRecord(c->ev_state, cs)) != hipSuccess) return e;
  c->ev_valid = true;
  if (cs != ks) return hipStreamWaitEvent(ks, c->ev_state, 0);
  return hipSuccess;
}

}  // namespace

namespace moe {

// the cached layer's residency step: the experts with kept rows in counts[E] (device)
hipError_t cache_enqueue_counts(moe_expert_cache* c, const int32_t* counts, hipStream_t cs,
                                hipStream_t ks) {
  return enqueue_residency(c, counts, nullptr, cs, ks);
}

}  // namespace moe

extern "C" {

size_t moe_cache_pool_bytes(const moe_dims_t* d, int32_t slots) {
  if (!cache_dims_ok(d, false) || slots < 1 || slots > kMaxSlots) return 0;
  return pool_layout(d, slots, false).total;
}

size_t moe_cache_pool_bytes_mxfp4(const moe_dims_t* d, int32_t slots) {
  if (!cache_dims_ok(d, true) || slots < 1 || slots > kMaxSlots) return 0;
  return pool_layout(d, slots, true).total;
}

}  // extern "C"

namespace {

// host arrays: w = the values (bf16) or codes (MXFP4), s = the MXFP4 scales (null for bf16)
moe_status_t cache_create(const moe_dims_t* d, int32_t slots, bool mx, const void* const w[3],
                          const void* const sc[3], void* pool, size_t pool_bytes,
                          moe_expert_cache_t** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (!d || slots < 1 || !w[0] || !w[1] || !w[2] || !pool) return MOE_ERR_INVALID_ARG;
  if (mx && (!sc[0] || !sc[1] || !sc[2])) return MOE_ERR_INVALID_ARG;
  if (!cache_dims_ok(d, mx) || slots > kMaxSlots) return MOE_ERR_UNSUPPORTED;
  const PoolLayout L = pool_layout(d, slots, mx);
  if (pool_bytes < L.total) return MOE_ERR_WORKSPACE;
  // the copy kernel reads the host arrays over PCIe: they must be pinned, device-visible
  const void* host[6] = {w[0], w[1], w[2], sc[0], sc[1], sc[2]};
  const void* visible[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  for (int i = 0; i < (mx ? 6 : 3); ++i) {
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, const_cast<void*>(host[i]), 0) != hipSuccess || !dp) {
      (void)hipGetLastError();  // clear the error the query left
      return MOE_ERR_INVALID_ARG;
    }
    visible[i] = dp;
  }
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return MOE_ERR_HIP;
  c->E = d->E;
  c->H = d->H;
  c->I = d->I;
  c->slots = slots;
  c->mx = mx;
  c->pool = (char*)pool;
  for (int i = 0; i < 6; ++i) c->part_off[i] = L.part[i];
  c->st.table = (int32_t*)(c->pool + L.table);
  c->st.owner = (int32_t*)(c->pool + L.owner);
  c->st.last_use = (int32_t*)(c->pool + L.last_use);
  c->st.copy_e = (int32_t*)(c->pool + L.copy_e);
  c->st.copy_s = (int32_t*)(c->pool + L.copy_s);
  c->st.stats = (int32_t*)(c->pool + L.stats);
  c->st.E = d->E;
  c->st.slots = slots;
  int64_t chunks = 0;
  c->expert_bytes = 0;
  for (int i = 0; i < 6; ++i) {
    c->copy.src[i] = (const char*)visible[i];
    c->copy.dst[i] = c->pool + L.part[i];
    c->copy.bytes[i] = (int64_t)L.part_bytes[i];
    c->copy.chunk_start[i] = chunks;
    chunks += (int64_t)L.part_bytes[i] / 16;
    c->expert_bytes += (int64_t)L.part_bytes[i];
  }
  c->copy.chunk_start[6] = chunks;
  c->state_ready = false;
  c->ev_valid = false;
  if (hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming) != hipSuccess) {
    delete c;
    return MOE_ERR_HIP;
  }
  if (hipEventCreateWithFlags(&c->ev_state, hipEventDisableTiming) != hipSuccess) {
    (void)hipEventDestroy(c->ev_compute);
    delete c;
    return MOE_ERR_HIP;
  }
  *out = c;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_cache_create(const moe_dims_t* d, int32_t slots, const void* host_w1,
                              const void* host_w3, const void* host_w2, void* pool,
                              size_t pool_bytes, moe_expert_cache_t** out) {
  const void* w[3] = {host_w1, host_w3, host_w2};
  const void* sc[3] = {nullptr, nullptr, nullptr};
  return cache_create(d, slots, false, w, sc, pool, pool_bytes, out);
}

moe_status_t moe_cache_create_mxfp4(const moe_dims_t* d, int32_t slots, const uint8_t* host_w1q,
                                    const uint8_t* host_w1s, const uint8_t* host_w3q,
                                    const uint8_t* host_w3s, const uint8_t* host_w2q,
                                    const uint8_t* host_w2s, void* pool, size_t pool_bytes,
                                    moe_expert_cache_t** out) {
  const void* w[3] = {host_w1q, host_w3q, host_w2q};
  const void* sc[3] = {host_w1s, host_w3s, host_w2s};
  return cache_create(d, slots, true, w, sc, pool, pool_bytes, out);
}

void moe_cache_destroy(moe_expert_cache_t* c) {
  if (!c) return;
  (void)hipEventDestroy(c->ev_compute);
  (void)hipEventDestroy(c->ev_state);
  delete c;
}

moe_status_t moe_cache_slots(const moe_expert_cache_t* c, int32_t* slot_of) {
  if (!c || !slot_of) return MOE_ERR_INVALID_ARG;
  if (!c->state_ready) {
    std::fill(slot_of, slot_of + c->E, -1);
    return MOE_OK;
  }
  if (c->ev_valid && hipEventSynchronize(c->ev_state) != hipSuccess) return MOE_ERR_HIP;
  if (hipMemcpy(slot_of, c->st.table, (size_t)c->E * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_cache_last_step(const moe_expert_cache_t* c, moe_cache_step_t* info) {
  if (!c || !info) return MOE_ERR_INVALID_ARG;
  *info = moe_cache_step_t{};
  if (!c->state_ready) return MOE_OK;
  if (c->ev_valid && hipEventSynchronize(c->ev_state) != hipSuccess) return MOE_ERR_HIP;
  int32_t s[ST_WORDS];
  if (hipMemcpy(s, c->st.stats, sizeof(s), hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  info->requested = s[ST_REQUESTED];
  info->hits = s[ST_HITS];
  info->loads = s[ST_LOADS];
  info->evictions = s[ST_EVICTIONS];
  info->bytes_loaded = (int64_t)s[ST_LOADS] * c->expert_bytes;
  return s[ST_STATUS] ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

moe_status_t moe_cache_load(moe_expert_cache_t* c, const int32_t* experts, int32_t n,
                            void* copy_stream, void* stream, moe_cache_step_t* info) {
  if (!c || n < 0 || (n > 0 && !experts)) return MOE_ERR_INVALID_ARG;
  std::vector<int32_t> need(experts, experts + n);
  for (int32_t e : need)
    if (e < 0 || e >= c->E) return MOE_ERR_INVALID_ARG;
  std::sort(need.begin(), need.end());
  need.erase(std::unique(need.begin(), need.end()), need.end());
  if ((int)need.size() > c->slots) return MOE_ERR_UNSUPPORTED;
  PlanRequest r;
  r.n = (int)need.size();
  for (int i = 0; i < r.n; ++i) r.ids[i] = (uint16_t)need[i];
  if (enqueue_residency(c, nullptr, &r, (hipStream_t)copy_stream, (hipStream_t)stream) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return info ? moe_cache_last_step(c, info) : MOE_OK;
}

}  // extern "C"
