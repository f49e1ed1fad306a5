"""Plain model of the expert cache's residency policy (pure Python, small cases).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's CPU-baseline
leg use this package.

"MoE 推理架构深度实战：从 Expert Parallelism 到 DeepSeek-V3 的工程落地" §3.2 keeps a subset of
the experts in HBM and loads the others from host memory on demand: before a batch, the experts
it needs are made resident, evicting the least recently used resident experts that the batch
does not need, and the missing ones are copied in.  Readings: "least recently used" is the
smallest step at which an expert was last requested (ties: lower expert id); an expert the
current batch requests is never evicted for it; a freed or never-used slot is reused lowest
slot first; missing experts are loaded in ascending id order.  A batch needing more experts than
there are slots is rejected.
"""
from __future__ import annotations


class LRUCache:
    def __init__(self, num_experts: int, slots: int):
        self.E = num_experts
        self.slots = slots
        self.slot_of = [-1] * num_experts   # expert -> slot, -1 when not resident
        self.expert_in = [-1] * slots       # slot -> expert, -1 when free
        self.last_use = [-1] * num_experts  # step of the last request
        self.step = 0

    def request(self, experts):
        """Make `experts` resident for one batch.  Returns (hits, loads, evictions): hits and
        loads as sorted expert lists, evictions as (expert, slot) pairs in eviction order."""
        need = sorted(set(int(e) for e in experts))
        if len(need) > self.slots:
            raise ValueError("batch needs more experts than there are slots")
        self.step += 1
        hits = [e for e in need if self.slot_of[e] >= 0]
        loads = [e for e in need if self.slot_of[e] < 0]
        for e in need:
            self.last_use[e] = self.step
        evictions = []
        for e in loads:
            free = [s for s in range(self.slots) if self.expert_in[s] < 0]
            if free:
                s = free[0]
            else:
                victims = [v for v in range(self.E) if self.slot_of[v] >= 0 and v not in need]
                v = min(victims, key=lambda v: (self.last_use[v], v))
                s = self.slot_of[v]
                self.slot_of[v] = -1
                self.expert_in[s] = -1
                evictions.append((v, s))
            self.slot_of[e] = s
            self.expert_in[s] = e
        return hits, loads, evictions
