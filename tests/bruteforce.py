"""Brute-force replay of the slot buffer, for tiny traces only.

Written independently of the oracle: it keeps, per slot, only the id it holds
and the step at which that id was last selected, and derives everything else
from those two numbers:
  - lifetime after step t of a slot last selected at step t' is
    max(L - (t - t'), 0) (reset to L on selection, minus one per later step,
    floored at 0);
  - LRU bucket at step t is min(floor((t - t' - 1) / W), B - 1), W steps per
    bucket.
Matching is an O(|U| * S) scan and each victim is found by a full-scan argmin
over the remaining candidates, one miss at a time.
"""
from __future__ import annotations


class BruteBuffer:
    def __init__(self, S, N, L, B, policy, W=1):
        self.S, self.N, self.L, self.B, self.policy, self.W = S, N, L, B, policy, W
        self.tok = [-1] * S
        self.last = [None] * S
        self.t = 0

    def life_array(self):
        """The caller-visible counter per slot after the last step."""
        out = []
        t = self.t - 1
        for s in range(self.S):
            if self.tok[s] < 0:
                out.append(-1 if self.policy == "lru" else 0)
            elif self.policy == "lru":
                out.append(self.last[s])
            else:
                out.append(max(self.L - (t - self.last[s]), 0))
        return out

    def _key(self, s, t):
        if self.tok[s] < 0:
            return (0, 0, s)
        age = t - self.last[s]
        if self.policy == "lru":
            return (1, -min((age - 1) // self.W, self.B - 1), s)
        return (1, max(self.L - age, 0), s)

    def step(self, lists):
        """lists: T sorted id lists.  Returns per-token (hit, slot) lists and counts."""
        t = self.t
        union = sorted(set(x for lst in lists for x in lst))
        assert len(union) <= self.S
        slot_of = {}
        hit = {}
        for x in union:
            found = [s for s in range(self.S) if self.tok[s] == x]
            assert len(found) <= 1
            hit[x] = bool(found)
            if found:
                slot_of[x] = found[0]
        held = set(slot_of.values())
        candidates = [s for s in range(self.S) if s not in held]
        evict = 0
        for x in union:                     # ascending id order
            if hit[x]:
                continue
            best = min(candidates, key=lambda s: self._key(s, t))
            candidates.remove(best)
            if self.tok[best] >= 0:
                evict += 1
            self.tok[best] = x
            slot_of[x] = best
        for x in union:
            self.last[slot_of[x]] = t
        self.t += 1
        flags = [[hit[x] for x in lst] for lst in lists]
        slots = [[slot_of[x] for x in lst] for lst in lists]
        n_hit = sum(hit.values())
        return flags, slots, dict(n_hit=n_hit, n_miss=len(union) - n_hit, n_evict=evict,
                                  n_union=len(union))
