"""Reference of the expert slot pool's replacement policy (LFU with recency).

TEST INFRASTRUCTURE ONLY: the test suite and the benchmark are its only
users; the library's pool (csrc/pool.hip) shares no code with it.

The pages keep hot routed experts in a bounded pool of slots and evict by LFU
combined with recency; hit rates of 43-70% are quoted (page "Paquets Swiftlet
80B Qwen ..." on xix.ai, 4th and 8th paragraphs; page "Swiftlet: 在 Mac 和
iPhone 上執行 80B 與 35B Qwen 模型" on agentlenshq.com, section
"記憶體管理與權重串流", item "LFU 快取").  They give no further rule; the
reading (P1-P4 in the design notes) is:

P1  a key is (layer, expert); one request (one layer call) names a list of
    experts of one layer, processed in the given order, and is one tick of
    the clock;
P2  a hit adds 1 to the key's use count and sets its last use to the tick;
P3  a miss loads the key into the lowest free slot, or else into the slot of
    the resident key with the smallest (use count, last use, slot) that the
    current request has not used; the new key starts with count 1 and last
    use = the tick; a repeated expert within a request is a hit;
P4  a request naming more distinct experts than there are slots is refused.
"""
from __future__ import annotations


class SlotPool:
    """Plain reference: dictionaries and linear scans."""

    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.slot_key = [None] * n_slots       # key held by each slot
        self.where = {}                        # key -> slot
        self.count = {}                        # key -> use count
        self.last = {}                         # key -> last use tick
        self.tick = 0
        self.hits = self.misses = self.evictions = 0

    def require(self, layer: int, experts) -> list:
        """Make the experts of `layer` resident.  Returns the (expert, slot)
        loads of this request in order (the misses)."""
        distinct = []
        for e in experts:
            if e not in distinct:
                distinct.append(e)
        if len(distinct) > self.n_slots:
            raise ValueError("more distinct experts than slots")
        self.tick += 1
        loads = []
        for e in experts:
            key = (layer, int(e))
            if key in self.where:
                self.hits += 1
                self.count[key] += 1
                self.last[key] = self.tick
                continue
            self.misses += 1
            free = [s for s in range(self.n_slots) if self.slot_key[s] is None]
            if free:
                slot = free[0]
            else:
                cands = [(self.count[k], self.last[k], s) for s, k in enumerate(self.slot_key)
                         if self.last[k] < self.tick]
                _, _, slot = min(cands)
                old = self.slot_key[slot]
                del self.where[old], self.count[old], self.last[old]
                self.evictions += 1
            self.slot_key[slot] = key
            self.where[key] = slot
            self.count[key] = 1
            self.last[key] = self.tick
            loads.append((int(e), slot))
        return loads

    def slot_of(self, layer: int, expert: int) -> int:
        return self.where.get((layer, int(expert)), -1)
