"""The shared expert-slot cache, one layer call at a time (oracle; test infrastructure).

What the pages fix:
* [FT] "语义感知专家缓存": one LRU residency space shared by every MoE layer;
  a hit refreshes the expert's recency, a fill admits a newly chosen expert,
  eviction takes the expert least recently needed.
* [FT] "FTW 权重格式与平台适配" and [FTK] (two-level memory paragraph): an
  expert's identity is the flat logical id l*E + e; one slot holds every
  tensor of one (layer, expert).
* [FT] "Device-side 缓存控制": per layer one pass does dedup of the routed
  experts -> hit/miss against the residency table -> the fill count q from
  the bandwidth ratio -> victim slots -> rewrite of each route to a physical
  slot or to a "run on host" flag; victims are the K least recently used
  slots found in one scan, of which the miss path takes the first q.
* [FT] "q* 策略": fills F (|F| = q) enter the cache and run on the GPU; the
  host set C runs from the host pool and leaves residency untouched; the
  choice of F is left to the replacement policy.
* [FT] "执行顺序与工程细节": GPU order is cache update, copy of F, grouped
  evaluation of G = H u F.

Readings adopted where the pages are silent (all listed in the design notes):
* dedup order and the hit / miss lists are ascending logical id;
* recency: one global tick per layer call; inside a call the touch order is
  the hits (ascending id) then the fills (ascending id), stamped
  (tick << 16) | (1 + rank); seeded slot i has stamp 1 + i, empty slots 0;
* slots holding a hit of this call are never victims (their bytes are read
  by the grouped evaluation after the copy), so q = min(q*, #non-hit slots);
* victims: ascending (stamp, slot) among non-hit, non-reserved slots; F is
  the first q misses by ascending id and fill i goes to victim i;
* slots reserved by the prefill double buffer are outside the LRU;
* on-demand loading (no room for the full-layer buffers) fills every miss
  that finds a non-hit slot: q* = m instead of the bandwidth split;
* at the end of prefill the experts the buffers hold become residents (see
  finish_prefill for the order of their stamps);
* a resize keeps the most recent residents that fit (see resize).
"""
import numpy as np

from .qsplit import q_star as _q_star

EMPTY = -1
RESERVED = -2


class StepResult:
    """Decisions of one layer call (plain lists / arrays, for comparison)."""

    __slots__ = ("uniq", "is_hit", "q_star", "q", "fill_id", "fill_slot", "fill_evicted",
                 "host_id", "pick_slot", "hits", "misses", "g_slots")

    def __repr__(self):
        return ("StepResult(u=%d, hits=%s, misses=%s, q*=%d, q=%d, fill=%s, host=%s)"
                % (len(self.uniq), self.hits, self.misses, self.q_star, self.q,
                   list(zip(self.fill_id, self.fill_slot, self.fill_evicted)), self.host_id))


class ExpertCache:
    def __init__(self, L: int, E: int, C: int, bp: int, bh: int):
        if C <= 0 or L <= 0 or E <= 0:
            raise ValueError("bad shape")
        self.L, self.E, self.C, self.bp, self.bh = L, E, C, bp, bh
        self.slot_id = [EMPTY] * C
        self.ts = [0] * C
        self.id_slot = [EMPTY] * (L * E)
        self.tick = 1
        # running counters: layer calls, unique, hits, misses, fills, host
        self.counters = dict(calls=0, uniq=0, hits=0, misses=0, fills=0, host=0)

    # -- set-up ---------------------------------------------------------------
    def seed(self, ids):
        """Slot i <- logical id ids[i], stamp 1 + i (older than any call)."""
        for i, lid in enumerate(ids):
            old = self.slot_id[i]
            if old >= 0:
                self.id_slot[old] = EMPTY
            self.slot_id[i] = int(lid)
            self.ts[i] = 1 + i
            self.id_slot[int(lid)] = i

    def reserve(self, first: int, count: int):
        """Take slots [first, first+count) out of the LRU (prefill buffers)."""
        for s in range(first, first + count):
            old = self.slot_id[s]
            if old >= 0:
                self.id_slot[old] = EMPTY
            self.slot_id[s] = RESERVED
            self.ts[s] = 0

    def release(self, first: int, count: int):
        for s in range(first, first + count):
            self.slot_id[s] = EMPTY
            self.ts[s] = 0

    def finish_prefill(self, first: int, n_buf: int, loaded):
        """End of prefill: the full-layer buffers hand what they hold to the
        decode cache.

        [FT] "全层双缓冲" and [FTK] (prefill paragraph): the buffers are slots
        of the one shared pool, so the experts they hold when prefill ends are
        the decode cache's first residents, with no copy and no separate
        hand-over phase.  Buffer b spans slots [first + b*E, first + b*E + E).
        loaded: (b, layer) for each buffer holding a complete layer, least
        recently loaded first.  Readings: a later load is more recent; inside
        a buffer, ascending expert index; expert e of the buffer at position
        pos of `loaded` gets stamp (tick << 16) | (1 + pos*E + e); an expert
        already resident in a decode slot keeps that slot, takes the new
        stamp, and its buffer slot is left empty; every other buffer slot is
        left empty; the tick then advances by one.
        """
        E = self.E
        self.release(first, n_buf * E)
        for pos, (b, layer) in enumerate(loaded):
            for e in range(E):
                lid = layer * E + e
                stamp = (self.tick << 16) | (1 + pos * E + e)
                old = self.id_slot[lid]
                if old >= 0:
                    self.ts[old] = stamp
                    continue
                s = first + b * E + e
                self.slot_id[s] = lid
                self.id_slot[lid] = s
                self.ts[s] = stamp
        self.tick += 1

    def resize(self, new_C: int):
        """Change the number of slots at a safe point between layer calls.

        [FTK] (safe-point paragraph) and [FT] (section "挑战三"): the memory
        budget is re-split at run time without a restart; the host pool is
        the ground truth, so a smaller GPU cache changes no output.  Readings:
        no slot may be reserved; the cache keeps its min(residents, new_C)
        most recent residents (largest (stamp, slot)) with their stamps; a
        kept resident whose slot is below new_C stays in it; the other kept
        residents move, in ascending order of their old slots, to the free
        slots below new_C (empty, or holding a resident that is dropped), in
        ascending order; slots added by growth are empty; tick and counters
        are unchanged.  Returns the moves as [(old slot, new slot)].
        """
        if new_C <= 0:
            raise ValueError("bad size")
        if RESERVED in self.slot_id:
            raise ValueError("slots are reserved")
        res = sorted((self.ts[s], s) for s in range(self.C) if self.slot_id[s] >= 0)
        keep = set(s for _, s in res[len(res) - min(len(res), new_C):])
        stay = [s for s in range(min(self.C, new_C)) if s in keep]
        movers = sorted(s for s in keep if s >= new_C)
        free = [s for s in range(new_C) if s not in keep]
        moves = list(zip(movers, free))
        slot_id = [EMPTY] * new_C
        ts = [0] * new_C
        for s in stay:
            slot_id[s], ts[s] = self.slot_id[s], self.ts[s]
        for src, dst in moves:
            slot_id[dst], ts[dst] = self.slot_id[src], self.ts[src]
        self.id_slot = [EMPTY] * (self.L * self.E)
        for s, lid in enumerate(slot_id):
            if lid >= 0:
                self.id_slot[lid] = s
        self.slot_id, self.ts, self.C = slot_id, ts, new_C
        return moves

    # -- one layer call --------------------------------------------------------
    def step(self, layer: int, ids, copy: bool = True, fill_all: bool = False) -> StepResult:
        """One layer call.  fill_all: on-demand loading ([FT] "全层双缓冲",
        the fallback when two full layers do not fit): every miss is a fill
        candidate, q* = m; q is still capped by the non-hit slots."""
        ids = np.asarray(ids, dtype=np.int64)
        T, k = ids.shape
        E = self.E
        if ids.size and (ids.min() < 0 or ids.max() >= E):
            raise ValueError("expert id out of range")
        logical = layer * E + ids

        uniq = sorted(set(int(v) for v in logical.reshape(-1)))
        hits = [i for i in uniq if self.id_slot[i] >= 0]
        misses = [i for i in uniq if self.id_slot[i] < 0]
        m = len(misses)
        qs = m if fill_all else _q_star(m, self.bp, self.bh)

        hit_slots = set(self.id_slot[i] for i in hits)
        cand = [s for s in range(self.C) if s not in hit_slots and self.slot_id[s] != RESERVED]
        cand.sort(key=lambda s: (self.ts[s], s))
        q = min(qs, len(cand))
        victims = cand[:q]
        fills = misses[:q]
        host = misses[q:]

        evicted = []
        for f, v in zip(fills, victims):
            old = self.slot_id[v]
            evicted.append(old)
            if old >= 0:
                self.id_slot[old] = EMPTY
            self.slot_id[v] = f
            self.id_slot[f] = v

        for rank, lid in enumerate(hits + fills):
            self.ts[self.id_slot[lid]] = (self.tick << 16) | (1 + rank)
        self.tick += 1

        gset = set(hits) | set(fills)
        pick_slot = np.full((T, k), -1, np.int32)
        for t in range(T):
            for j in range(k):
                lid = int(logical[t, j])
                if lid in gset:
                    pick_slot[t, j] = self.id_slot[lid]

        c = self.counters
        c["calls"] += 1
        c["uniq"] += len(uniq)
        c["hits"] += len(hits)
        c["misses"] += m
        c["fills"] += q
        c["host"] += len(host)

        r = StepResult()
        r.uniq = uniq
        r.is_hit = [1 if i in set(hits) else 0 for i in uniq]
        r.q_star, r.q = qs, q
        r.fill_id, r.fill_slot, r.fill_evicted = fills, victims, evicted
        r.host_id = host
        r.pick_slot = pick_slot
        r.hits, r.misses = hits, misses
        r.g_slots = [self.id_slot[i] for i in hits + fills]
        return r

    # -- views -----------------------------------------------------------------
    def tables(self):
        return (np.array(self.slot_id, np.int32), np.array(self.ts, np.uint64),
                np.array(self.id_slot, np.int32), self.tick)
