"""Pins for oracle/ring.py: printed page values, the concat-and-prune manager,
a literal ring simulation, and the window boundary rule."""

import os
import random

import pytest

from oracle.ring import (concat_prune, resident_positions, simulate_appends, slot_contents,
                         slot_of)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _held(table):
    return sorted(p for p in table if p >= 0)


def test_demo_trace_w4():
    """[ring] §4.3: printed visible positions and used-slot counts, W = 4."""
    rows = _read("ring_demo_w4.txt")
    steps = [r for r in rows if r[0].isdigit()]
    assert len(steps) == 10
    for step, new_pos, visible, used in steps:
        t = int(step)
        assert int(new_pos) == t
        want = [int(x) for x in visible.split(",")]
        table = simulate_appends(range(t + 1), 0, 4)
        assert _held(table) == want
        assert sum(p >= 0 for p in table) == int(used)
        assert resident_positions(t, 0, 4) == want
        assert slot_contents(t, 0, 4) == table
    final = {r[0]: [int(x) for x in r[1].split(",")] for r in rows if not r[0].isdigit()}
    table = simulate_appends(range(10), 0, 4)
    assert _held(table) == final["final_positions"]
    # entry k of the demo is written by the k-th append, so its insert
    # sequence number is the position it holds
    assert _held(table) == final["final_insert_seq"]


def test_capacity4_abcdef():
    """[ring] §1.4: E lands in A's slot, F in B's, the ring holds C..F."""
    rows = {r[0]: r[1:] for r in _read("ring_capacity4.txt")}
    cap = int(rows["capacity"][0])
    names = rows["writes"][0].split(",")
    index = {n: i for i, n in enumerate(names)}
    for line in [r for r in _read("ring_capacity4.txt") if r[0] == "same_slot"]:
        a, b = line[1], line[2]
        assert slot_of(index[a], 0, cap) == slot_of(index[b], 0, cap)
    table = simulate_appends(range(len(names)), 0, cap)
    assert sorted(names[p] for p in table if p >= 0) == rows["held"][0].split(",")


SW = [(0, 4), (4, 16), (1, 2), (4, 4), (2, 7), (0, 1), (3, 1), (4, 5)]


@pytest.mark.parametrize("sinks,window", SW)
def test_concat_prune_equals_set_definition(sinks, window):
    """[sink] manager (concat, then keep first S and last W) vs the closed form,
    one token per call, for every t <= 200."""
    for t in range(201):
        got = concat_prune([[p] for p in range(t + 1)], sinks, window)
        assert got == resident_positions(t, sinks, window), (t, got)


@pytest.mark.parametrize("sinks,window", SW)
def test_concat_prune_chunked_calls(sinks, window):
    """Multi-token calls prune to the same set as single-token calls."""
    rng = random.Random(1000 * sinks + window)
    for _ in range(30):
        t = rng.randrange(0, 150)
        calls, p = [], 0
        while p <= t:
            n = min(rng.randrange(1, 3 * (sinks + window) + 2), t + 1 - p)
            calls.append(list(range(p, p + n)))
            p += n
        assert concat_prune(calls, sinks, window) == resident_positions(t, sinks, window)


@pytest.mark.parametrize("sinks,window", SW)
def test_slot_contents_closed_form_vs_simulation(sinks, window):
    for t in range(5 * (sinks + window) + 1):
        table = simulate_appends(range(t + 1), sinks, window)
        assert slot_contents(t, sinks, window) == table, t
        assert _held(table) == resident_positions(t, sinks, window), t


@pytest.mark.parametrize("sinks,window", SW)
def test_window_boundary(sinks, window):
    """[ring] §6: earliest visible is t-W+1, never t-W; cover t < W and t >= W."""
    for t in list(range(0, window + 1)) + [window + 5, 3 * window + 1]:
        r = resident_positions(t, sinks, window)
        assert t in r
        assert max(0, t - window + 1) in r
        if t - window >= sinks:
            assert t - window not in r
        assert len(r) == min(t + 1, sinks + window)


def test_sinks_kept_forever():
    for t in (19, 20, 100, 10_000):
        r = resident_positions(t, 4, 16)
        assert r[:4] == [0, 1, 2, 3]
        assert r[4:] == list(range(t - 15, t + 1))


def test_ring_memory_stays_at_window():
    """[ring] §4.4: 10,000 tokens with W = 1024: the ring holds 1024 entries,
    an append-only list holds 10,000."""
    table = simulate_appends(range(10_000), 0, 1024)
    assert sum(p >= 0 for p in table) == 1024
    assert len(table) == 1024
    naive = list(range(10_000))
    assert len(naive) == 10_000


def test_negative_position_rejected():
    with pytest.raises(ValueError):
        slot_of(-1, 4, 16)


def test_pins_catch_planted_mistakes():
    """Each plausible slip in the ring oracle fails one of the pins above."""

    def window_off_by_one(t, s, w):            # keeps t-W as well
        return sorted(set(range(min(s, t + 1))) | set(range(max(0, t - w), t + 1)))

    def sinks_dropped(t, s, w):                # pure window
        return sorted(set(range(max(0, t - w + 1), t + 1)))

    def window_excludes_current(t, s, w):      # attends before appending
        return sorted(set(range(min(s, t + 1))) | set(range(max(0, t - w), t)))

    for bad in (window_off_by_one, sinks_dropped, window_excludes_current):
        caught = any(bad(t, s, w) != concat_prune([[p] for p in range(t + 1)], s, w)
                     for s, w in SW for t in range(40))
        assert caught, bad.__name__

    def slot_off_by_one(p, s, w):              # ring index shifted by one
        return p if p < s else s + (p + 1) % w

    assert not all(slot_off_by_one(step, 0, w) == slot
                   for step, w, slot in _slot_rule_examples())


def _slot_rule_examples():
    return [(int(a), int(b), int(c)) for tag, a, b, c in
            (r for r in _read("ring_capacity4.txt") if r[0] == "step_window_slot")]


def test_slot_rule_without_sinks():
    """[ring] §5.1: with no sinks the physical slot of decode step k is k mod W
    (positions equal step numbers in the demo)."""
    ex = _slot_rule_examples()
    assert ex
    for step, w, slot in ex:
        assert slot_of(step, 0, w) == slot
