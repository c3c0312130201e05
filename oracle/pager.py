"""Which VRAM slot holds which expert, step by step: the slot-miss path's
replacement rule.

vllm-expert-pager article (rand.pepabo.com), "hierarchical paging of expert
weights": every MoE layer has its own VRAM slots, one expert per slot, and
the tier is managed least-recently-used; an expert that a step needs and
VRAM does not hold is copied in from host RAM. Readings taken where the page
is silent: a step's misses are placed in ascending expert id; a miss takes
the free slot with the lowest index, else the slot of the resident expert,
not needed by this step, whose last use is oldest (ties to the lower expert
id); after the step every expert it needed counts as used at that step. A
step that needs more distinct experts than the layer has slots is refused
(the page switches such a step to a working buffer holding them all).
"""


class LRUSlots:
    def __init__(self, E: int, n_slots: int):
        self.E, self.n_slots = E, n_slots
        self.slot_of = [-1] * E
        self.owner = [-1] * n_slots
        self.last = [-1] * E
        self.step = 0
        self.hits = self.misses = 0

    def plan(self, needed):
        """Returns (table [E] list, fills [(expert, slot)] in ascending expert id)."""
        want = sorted({int(e) for e in needed if 0 <= int(e) < self.E})
        if len(want) > self.n_slots:
            raise ValueError("more distinct experts than slots")
        wanted = set(want)
        fills = []
        for e in want:
            if self.slot_of[e] >= 0:
                self.hits += 1
                continue
            self.misses += 1
            free = [s for s in range(self.n_slots) if self.owner[s] < 0]
            if free:
                slot = free[0]
            else:
                victim = min((v for v in range(self.E) if self.slot_of[v] >= 0 and v not in wanted),
                             key=lambda v: (self.last[v], v))
                slot = self.slot_of[victim]
                self.slot_of[victim] = -1
            self.slot_of[e] = slot
            self.owner[slot] = e
            fills.append((e, slot))
        for e in want:
            self.last[e] = self.step
        self.step += 1
        return list(self.slot_of), fills
