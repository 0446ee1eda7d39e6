"""Which positions a sink + sliding-window cache holds, and where.

Definitions followed:

* Window: at position t the visible positions are t-W+1 .. t; t-W is the
  classic off-by-one ([ring] §2.2 and §6, boundary advice).
* Sinks: the first S positions are kept forever next to the window; the
  cache is [K_0..K_{S-1}] united with [K_{t-W+1}..K_t] ([sink], the
  StreamingLLM cache formula with S = 4).
* Ring: a fixed number of slots, each new entry overwrites the oldest one
  ([ring] §1.4 and §3.3, head = (head + 1) mod W).

Pins (tests/test_oracle_ring.py): the printed demo trace and the capacity-4
A..F example of [ring] (golden fixtures; with S = 0 they fix the slot of every
position, since the page's ring writes entry number k into slot k mod W), the
concat-and-prune manager of [sink] run on position lists, and a literal
sequential ring simulation.

The slot index of a position (`slot_of`) is a reading: sinks sit in slots
0..S-1 and a later position p goes to slot S + (p mod W), i.e. "pos mod W
behind pinned sink slots".  With S = 0 it is exactly the [ring] demo's
head pointer; for S > 0 only the set of held positions is pinned by the pages.
"""

from __future__ import annotations


def slot_of(p: int, sinks: int, window: int) -> int:
    """Cache slot of absolute position p (p >= 0)."""
    if p < 0:
        raise ValueError("position must be non-negative")
    if p < sinks:
        return p
    return sinks + p % window


def resident_positions(t: int, sinks: int, window: int) -> list:
    """R(t): positions held after positions 0..t were appended, ascending.

    Plain set definition: {0 .. min(S, t+1)-1} united with {max(0, t-W+1) .. t}."""
    sink_set = set(range(0, min(sinks, t + 1)))
    window_set = set(range(max(0, t - window + 1), t + 1))
    return sorted(sink_set | window_set)


def slot_contents(t: int, sinks: int, window: int) -> list:
    """Position held by every slot after positions 0..t were appended (-1 = empty).

    Closed form: sink slot s holds s once s <= t.  Ring slot S + r holds the
    latest appended position p >= S with p mod W == r, namely
    p* = t - ((t - r) mod W), if p* >= S."""
    table = [-1] * (sinks + window)
    for s in range(sinks):
        table[s] = s if s <= t else -1
    for r in range(window):
        p_star = t - ((t - r) % window)
        table[sinks + r] = p_star if p_star >= sinks else -1
    return table


def simulate_appends(positions, sinks: int, window: int, table=None) -> list:
    """Literal sequential ring: write each position into its slot, in order."""
    if table is None:
        table = [-1] * (sinks + window)
    for p in positions:
        table[slot_of(int(p), sinks, window)] = int(p)
    return table


def concat_prune(appends, sinks: int, window: int) -> list:
    """The [sink] page's cache manager, run on position lists.

    Each call concatenates the new positions; when the cache is longer than
    S + W it keeps the first S and the last W entries.  (The page's listing
    skips pruning on its very first call; the pruning rule is applied on
    every call here, which is what its capacity formula states.)"""
    cache: list = []
    for new in appends:
        cache = cache + list(new)
        if len(cache) > sinks + window:
            cache = cache[:sinks] + (cache[-window:] if window > 0 else [])
    return cache
