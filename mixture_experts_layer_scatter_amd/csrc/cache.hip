// Expert cache: the routed experts' weights resident in HBM up to a number of slots.
//
// "MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地" §3.2 keeps a
// subset of the experts in HBM and loads the others from host memory before a
// batch needs them, evicting the least recently used, with the copies on a
// separate stream so they can overlap compute.  Here the pool (W1, W3, W2 per
// slot, and the device expert -> slot table) is caller-allocated device memory, holding the
// experts in the layer's bf16 or as MXFP4 codes and scales (§5.2 of the same page serves with
// the expert cache and 4-bit experts together, so a slot then costs a quarter of the bytes);
// this file holds the host-side residency bookkeeping, the copies and the
// table updates.  The grouped GEMMs read expert e's weights from slot table[e]
// (GroupedGemm::group_slot).
//
// Residency policy: recency = the last batch that requested an expert (ties:
// lower id); a batch's own experts are never evicted for it; free slots are
// taken lowest first; missing experts load in ascending id order.
#include "../../include/moe.h"
#include "common.hpp"

#include <algorithm>
#include <new>
#include <vector>

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Pool: W1, W3, W2 slots (bf16 values or MXFP4 codes), then (MXFP4) their scale slots, then
// the table.  An MXFP4 expert's codes and scales are each one contiguous block, as
// moe_quantize_mxfp4 writes them for [E * I, H] and [E * H, I].
struct PoolLayout {
  size_t w1, w3, w2, s1, s3, s2, table, total;
  size_t code_13, code_2, scale_13, scale_2;  // bytes of one expert
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
  L.code_13 = L.code_2 = mx ? n / 2 : n * 2;
  L.scale_13 = L.scale_2 = mx ? n / 32 : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.w1 = take((size_t)slots * L.code_13);
  L.w3 = take((size_t)slots * L.code_13);
  L.w2 = take((size_t)slots * L.code_2);
  L.s1 = take((size_t)slots * L.scale_13);
  L.s3 = take((size_t)slots * L.scale_13);
  L.s2 = take((size_t)slots * L.scale_2);
  L.table = take((size_t)d->E * 4);
  L.total = o;
  return L;
}

// expert -> slot table changes, passed by value (no host buffer has to outlive the launch)
constexpr int kMaxUpdates = 240;
struct TableUpdate {
  int n;
  int init_E;  // > 0: first set all init_E entries to -1
  int32_t expert[kMaxUpdates];
  int32_t slot[kMaxUpdates];
};

__global__ __launch_bounds__(256) void cache_table_kernel(int32_t* table, TableUpdate u) {
  for (int i = threadIdx.x; i < u.init_E; i += blockDim.x) table[i] = -1;
  __syncthreads();
  for (int i = threadIdx.x; i < u.n; i += blockDim.x) table[u.expert[i]] = u.slot[i];
}

}  // namespace

struct moe_expert_cache {
  int E, H, I, slots;
  bool mx;  // MXFP4 codes and scales (else bf16 values)
  const char *hw1, *hw3, *hw2, *hs1, *hs3, *hs2;
  char *pw1, *pw3, *pw2, *ps1, *ps3, *ps2;
  int32_t* table;
  size_t bytes13, bytes2, sbytes13, sbytes2;
  std::vector<int32_t> slot_of, expert_in;
  std::vector<int64_t> last_use;
  int64_t step;
  bool table_ready;
  bool copies_issued;  // ev_copies covers every copy this cache has enqueued so far
  hipEvent_t ev_compute, ev_copies;
};

namespace moe {

CacheView cache_view(const moe_expert_cache* c) {
  CacheView v;
  v.w1 = c->pw1;
  v.w3 = c->pw3;
  v.w2 = c->pw2;
  v.s1 = (const uint8_t*)c->ps1;
  v.s3 = (const uint8_t*)c->ps3;
  v.s2 = (const uint8_t*)c->ps2;
  v.mx = c->mx;
  v.table = c->table;
  v.E = c->E;
  v.H = c->H;
  v.I = c->I;
  return v;
}

}  // namespace moe

extern "C" {

size_t moe_cache_pool_bytes(const moe_dims_t* d, int32_t slots) {
  if (!cache_dims_ok(d, false) || slots < 1) return 0;
  return pool_layout(d, slots, false).total;
}

size_t moe_cache_pool_bytes_mxfp4(const moe_dims_t* d, int32_t slots) {
  if (!cache_dims_ok(d, true) || slots < 1) return 0;
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
  if (!cache_dims_ok(d, mx)) return MOE_ERR_UNSUPPORTED;
  const PoolLayout L = pool_layout(d, slots, mx);
  if (pool_bytes < L.total) return MOE_ERR_WORKSPACE;
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return MOE_ERR_HIP;
  c->E = d->E;
  c->H = d->H;
  c->I = d->I;
  c->slots = slots;
  c->mx = mx;
  c->hw1 = (const char*)w[0];
  c->hw3 = (const char*)w[1];
  c->hw2 = (const char*)w[2];
  c->hs1 = (const char*)sc[0];
  c->hs3 = (const char*)sc[1];
  c->hs2 = (const char*)sc[2];
  c->pw1 = (char*)pool + L.w1;
  c->pw3 = (char*)pool + L.w3;
  c->pw2 = (char*)pool + L.w2;
  c->ps1 = mx ? (char*)pool + L.s1 : nullptr;
  c->ps3 = mx ? (char*)pool + L.s3 : nullptr;
  c->ps2 = mx ? (char*)pool + L.s2 : nullptr;
  c->table = (int32_t*)((char*)pool + L.table);
  c->bytes13 = L.code_13;
  c->bytes2 = L.code_2;
  c->sbytes13 = L.scale_13;
  c->sbytes2 = L.scale_2;
  c->slot_of.assign(d->E, -1);
  c->expert_in.assign(slots, -1);
  c->last_use.assign(d->E, -1);
  c->step = 0;
  c->table_ready = false;
  c->copies_issued = false;
  if (hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming) != hipSuccess) {
    delete c;
    return MOE_ERR_HIP;
  }
  if (hipEventCreateWithFlags(&c->ev_copies, hipEventDisableTiming) != hipSuccess) {
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
  (void)hipEventDestroy(c->ev_copies);
  delete c;
}

moe_status_t moe_cache_slots(const moe_expert_cache_t* c, int32_t* slot_of) {
  if (!c || !slot_of) return MOE_ERR_INVALID_ARG;
  std::copy(c->slot_of.begin(), c->slot_of.end(), slot_of);
  return MOE_OK;
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

  // residency decisions on copies of the bookkeeping; committed once everything is enqueued
  std::vector<int32_t> slot_of = c->slot_of, expert_in = c->expert_in;
  std::vector<int64_t> last_use = c->last_use;
  const int64_t step = c->step + 1;
  std::vector<char> requested(c->E, 0);
  int hits = 0;
  std::vector<int32_t> loads;
  for (int32_t e : need) {
    requested[e] = 1;
    if (slot_of[e] >= 0) ++hits;
    else loads.push_back(e);
    last_use[e] = step;
  }
  std::vector<int32_t> upd_e, upd_s;  // table changes: evictions, then loads
  std::vector<std::pair<int32_t, int32_t>> placed;  // (expert, slot) to copy
  int evictions = 0;
  for (int32_t e : loads) {
    int s = -1;
    for (int i = 0; i < c->slots; ++i)
      if (expert_in[i] < 0) {
        s = i;
        break;
      }
    if (s < 0) {
      int victim = -1;
      for (int v = 0; v < c->E; ++v) {
        if (slot_of[v] < 0 || requested[v]) continue;
        if (victim < 0 || last_use[v] < last_use[victim]) victim = v;  // ties: lower id (first)
      }
      s = slot_of[victim];
      slot_of[victim] = -1;
      expert_in[s] = -1;
      upd_e.push_back(victim);
      upd_s.push_back(-1);
      ++evictions;
    }
    slot_of[e] = s;
    expert_in[s] = e;
    upd_e.push_back(e);
    upd_s.push_back(s);
    placed.push_back({e, s});
  }

  hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)stream;
  const bool same = cs == ks;
  if (!placed.empty()) {
    // slots about to be overwritten may still be read by earlier work on the compute stream;
    // copies of earlier calls (perhaps on another copy stream) go first
    if (!same) {
      if (hipEventRecord(c->ev_compute, ks) != hipSuccess) return MOE_ERR_HIP;
      if (hipStreamWaitEvent(cs, c->ev_compute, 0) != hipSuccess) return MOE_ERR_HIP;
    }
    if (c->copies_issued && hipStreamWaitEvent(cs, c->ev_copies, 0) != hipSuccess)
      return MOE_ERR_HIP;
    for (auto [e, s] : placed) {
      if (hipMemcpyAsync(c->pw1 + (size_t)s * c->bytes13, c->hw1 + (size_t)e * c->bytes13,
                         c->bytes13, hipMemcpyHostToDevice, cs) != hipSuccess ||
          hipMemcpyAsync(c->pw3 + (size_t)s * c->bytes13, c->hw3 + (size_t)e * c->bytes13,
                         c->bytes13, hipMemcpyHostToDevice, cs) != hipSuccess ||
          hipMemcpyAsync(c->pw2 + (size_t)s * c->bytes2, c->hw2 + (size_t)e * c->bytes2,
                         c->bytes2, hipMemcpyHostToDevice, cs) != hipSuccess)
        return MOE_ERR_HIP;
      if (c->mx &&
          (hipMemcpyAsync(c->ps1 + (size_t)s * c->sbytes13, c->hs1 + (size_t)e * c->sbytes13,
                          c->sbytes13, hipMemcpyHostToDevice, cs) != hipSuccess ||
           hipMemcpyAsync(c->ps3 + (size_t)s * c->sbytes13, c->hs3 + (size_t)e * c->sbytes13,
                          c->sbytes13, hipMemcpyHostToDevice, cs) != hipSuccess ||
           hipMemcpyAsync(c->ps2 + (size_t)s * c->sbytes2, c->hs2 + (size_t)e * c->sbytes2,
                          c->sbytes2, hipMemcpyHostToDevice, cs) != hipSuccess))
        return MOE_ERR_HIP;
    }
    if (hipEventRecord(c->ev_copies, cs) != hipSuccess) return MOE_ERR_HIP;
    c->copies_issued = true;
  }
  // the compute stream waits for every copy so far: resident experts whose copies an earlier
  // call enqueued may still be in flight
  if (c->copies_issued && hipStreamWaitEvent(ks, c->ev_copies, 0) != hipSuccess) return MOE_ERR_HIP;
  // table changes on the compute stream, after the copies it now waits for
  size_t i = 0;
  bool init = !c->table_ready;
  while (init || i < upd_e.size()) {
    TableUpdate u;
    u.init_E = init ? c->E : 0;
    u.n = 0;
    for (; i < upd_e.size() && u.n < kMaxUpdates; ++i, ++u.n) {
      u.expert[u.n] = upd_e[i];
      u.slot[u.n] = upd_s[i];
    }
    cache_table_kernel<<<1, 256, 0, ks>>>(c->table, u);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    init = false;
  }
  c->table_ready = true;
  c->slot_of.swap(slot_of);
  c->expert_in.swap(expert_in);
  c->last_use.swap(last_use);
  c->step = step;
  if (info) {
    info->requested = (int32_t)need.size();
    info->hits = hits;
    info->loads = (int32_t)placed.size();
    info->evictions = evictions;
    info->bytes_loaded = (int64_t)placed.size() *
                         (int64_t)(2 * c->bytes13 + c->bytes2 + 2 * c->sbytes13 + c->sbytes2);
  }
  return MOE_OK;
}

}  // extern "C"
