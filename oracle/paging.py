"""Which logical blocks a fixed device pool holds under LRU residency.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path imports this module.

[pool] ("paging", "residency policy"): a sequence's history lives in host
memory as 64-token blocks; the device keeps a fixed number of slots, each
holding one block plus a validity bit, and blocks move between the two on
demand.  Of the page's residency policies only LRU needs no trained model:
it assumes that what was used most recently matters most and evicts the
block used longest ago.  Blocks inside a sliding window must stay resident;
a caller expresses that by naming the window's blocks in every request.

Readings where the page is silent (each is stated in the functions below):

* A "use" of a block is being named in a request.  All blocks of one request
  are used at the same instant (the request's index).
* A missing block takes the lowest-numbered empty slot; with none left it
  takes the slot of the resident block with the oldest last use, ties going
  to the lower slot number.
* Blocks named by the request being served and by the one before it are
  never evicted: the decode step that the previous request prepared runs
  while the next request's blocks are copied in (the page overlaps the
  copies with the attention kernel), and it must find every block it named.
  A request that cannot be met that way is refused and leaves the pool as
  it was.
* Blocks are brought in for the next decode step while the current one runs:
  between `advance(N)` and the following advance (or `commit`) the blocks
  being copied are not yet visible and the slots they overwrite are already
  invisible.  `visible()` is the set a decode step sees at that moment.

Pins (tests/test_oracle_paging.py): for requests of one block each the pool
holds exactly the C most recently used distinct blocks (the defining
property of LRU, computed directly from the request string); the inclusion
property (a pool of C slots holds a subset of what C + 1 slots hold);
streaming a history in chunks of k blocks with C a multiple of k leaves the
last C / k chunks, block j in slot j mod C; invariants (no protected block
evicted, every requested block resident after the request, refusal leaves
the state unchanged) checked against brute force over random traces.
"""

from __future__ import annotations


class PoolRefused(ValueError):
    """A request that the pool cannot meet without evicting a protected block."""


class LruPool:
    """One sequence's pool of `capacity` slots."""

    def __init__(self, capacity: int):
        if capacity < 1:
            raise ValueError("capacity must be >= 1")
        self.capacity = capacity
        self.slot_block = [-1] * capacity   # logical block held by each slot
        self.last_use: dict = {}            # block -> index of the last request naming it
        self.clock = 0                      # index of the next request
        self.prev: set = set()              # blocks of the previous request
        self.loading: list = []             # (slot, block) copied in, not yet visible
        self.evicting: list = []            # (slot, block) evicted by the last request

    def resident(self) -> set:
        return {b for b in self.slot_block if b >= 0}

    def visible(self) -> set:
        """Blocks a decode step sees now: resident, minus blocks still being
        copied in; the slots evicted by the last request are already gone."""
        loading = {b for _, b in self.loading}
        return {b for b in self.slot_block if b >= 0 and b not in loading}

    def advance(self, request) -> list:
        """Serve one request; returns the (slot, block) loads it starts.

        Makes every named block resident, choosing victims by LRU among the
        blocks named neither now nor by the previous request."""
        req = list(dict.fromkeys(int(b) for b in request))  # first occurrence order
        protected = set(req) | self.prev
        slot_of = {b: s for s, b in enumerate(self.slot_block) if b >= 0}
        missing = [b for b in req if b not in slot_of]
        free = [s for s, b in enumerate(self.slot_block) if b < 0]
        evictable = [s for s, b in enumerate(self.slot_block) if b >= 0 and b not in protected]
        if len(missing) > len(free) + len(evictable):
            raise PoolRefused(f"{len(missing)} blocks missing, {len(free)} free slots and "
                              f"{len(evictable)} evictable blocks")
        # the previous request's copies become visible (its commit)
        self.loading = []
        self.evicting = []
        # LRU order of the evictable blocks: oldest use first, then lower slot
        evictable.sort(key=lambda s: (self.last_use[self.slot_block[s]], s))
        loads = []
        for b in missing:
            if free:
                s = free.pop(0)
            else:
                s = evictable.pop(0)
                self.evicting.append((s, self.slot_block[s]))
            self.slot_block[s] = b
            loads.append((s, b))
        for b in req:
            self.last_use[b] = self.clock
        self.clock += 1
        self.prev = set(req)
        self.loading = list(loads)
        return loads

    def commit(self) -> None:
        """The copies in flight become visible."""
        self.loading = []

    def request(self, request) -> list:
        """A request whose blocks are visible when it returns (advance + commit)."""
        loads = self.advance(request)
        self.commit()
        return loads

