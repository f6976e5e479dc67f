"""Brute-force model of one KV source, for pinning the CPU reference on tiny inputs.

Written separately from the reference and in another style: places are sets
of row positions built by enumeration, the hot cache is a list of
(row, stamp) pairs searched with dicts, victims come from sorting every
(stamp, slot) pair, and payload is tracked as (layer, pos) labels instead of
bytes.  It follows the same statement of the method (the resolution order,
the B-slot hot cache with least-recently-used replacement, host refill) and
the same readings of what the statement leaves open.
"""
from __future__ import annotations

OK, E_RANGE, E_CAPACITY, E_NO_HOST_COPY = 0, -2, -3, -4
FRESH = 1 << 29  # hot-cache location: the row was copied from host in this call


class BruteSource:
    def __init__(self, H, P, T, B, page_map, host_valid, n_layers=1):
        self.H, self.P, self.T, self.B = H, P, T, B
        self.page_map = list(page_map)
        self.host_valid = list(host_valid)
        self.L = H
        self.clock = 0
        self.slots = [(-1, 0)] * B
        self.n_layers = n_layers
        # payload labels: what each place holds, per layer
        self.tail = {l: {pos % T: pos for pos in range(max(0, H - T), H)} if T else {}
                     for l in range(n_layers)}
        self.hot = {l: {} for l in range(n_layers)}

    def ready_rows(self):
        full = self.H // self.P
        return {pos for pg in range(full) if self.page_map[pg] >= 0
                for pos in range(pg * self.P, (pg + 1) * self.P)}

    def tail_rows(self):
        return set(range(max(0, self.L - self.T), self.L)) if self.T else set()

    def append(self):
        pos = self.L
        if self.T:
            for l in range(self.n_layers):
                self.tail[l][pos % self.T] = pos
        self.L += 1

    def resolve(self, sel, fill_layer=0):
        """Returns (status, loc list of (place, index), fills list of (row, slot))."""
        if any(not (0 <= p < self.L) for p in sel):
            return E_RANGE, None, []
        now = self.clock + 1
        tail, ready = self.tail_rows(), self.ready_rows()
        pending = sorted({p for p in sel if p not in tail and p not in ready})
        where = {row: b for b, (row, _) in enumerate(self.slots) if row >= 0}
        hits = {u: where[u] for u in pending if u in where}
        misses = [u for u in pending if u not in where]
        if len(hits) + len(misses) > self.B:
            return E_CAPACITY, None, []
        for u in misses:
            if u < self.H and not self.host_valid[u // self.P]:
                return E_NO_HOST_COPY, None, []
        hit_slots = set(hits.values())
        order = sorted((st, b) for b, (_, st) in enumerate(self.slots) if b not in hit_slots)
        victims = [b for _, b in order[:len(misses)]]
        slots = list(self.slots)
        for u, b in hits.items():
            slots[b] = (u, now)
        for u, b in zip(misses, victims):
            slots[b] = (u, now)
        self.slots = slots
        self.clock = now
        fills = list(zip(misses, victims))
        if fill_layer >= 0:
            for u, b in fills:
                self.hot[fill_layer][b] = u
        place = {u: b for b, (u, _) in enumerate(slots) if u >= 0}
        loc = []
        for p in sel:
            if p in tail:
                loc.append((0, p % self.T))
            elif p in ready:
                pg = p // self.P
                loc.append((1, self.page_map[pg] * self.P + p % self.P))
            else:
                # rows copied from host in this call carry the fresh flag
                fresh = FRESH if p in misses else 0
                loc.append((2, place[p] | fresh))
        return OK, loc, fills

    def replay(self, layer, fills):
        for u, b in fills:
            self.hot[layer][b] = u

    def label(self, layer, place, index):
        """Row position whose payload a location should hold (pages: by owner)."""
        if place == 0:
            return self.tail[layer][index]
        if place == 2:
            return self.hot[layer][index & ~FRESH]
        phys, off = divmod(index, self.P)
        return self.page_map.index(phys) * self.P + off

    def tags(self):
        return [row for row, _ in self.slots]

    def stamps(self):
        return [st for _, st in self.slots]
