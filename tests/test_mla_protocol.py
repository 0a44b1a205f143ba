"""Host model of the hand-off protocol of the MLA split kernel (race detection).

The persistent MLA split kernel runs three roles in one workgroup that meet
only through LDS counters: two fetching waves move items (a segment's absorbed
query, then its 32-position tiles) into a 4-buffer ring, two score waves turn a
tile into P (each writing its 8 heads' rows of one of two P buffers) and four
P.V waves multiply P by the tile. Every wave runs at its own pace, so the only
thing that keeps a buffer from being refilled before every reader is done is
the counters' wait conditions.

This model restates those conditions (the fetch publishing landed items before
waiting for a free buffer, the first two items a step early; per-buffer
cumulative read counts of the ring; per-buffer written / read counts of the P
buffers) and runs the roles as coroutines under many random schedules, with
every DMA landing after a random delay. It checks that every wave reads the
item it expects from a buffer that holds it (both fetching waves' halves
landed), that P of tile k is complete when a P.V wave reads it and is not
overwritten before every P.V wave has read it, and that every schedule ends.

The same model with one read count for the whole ring and one written / read
count for both P buffers (sums over waves) shows the race those sums allowed:
fast waves' counts standing in for a slow wave's.
"""
from __future__ import annotations

import random

import pytest

RING, KSCORE, KPV, KFETCH = 4, 2, 4, 2
KWAVES = KSCORE + KPV
END = "end"


class Violation(Exception):
    pass


def items_of(rng: random.Random):
    """An item stream: segments of one q~ item followed by 1..6 tiles."""
    items = []
    for _ in range(rng.randint(1, 5)):
        items.append("q")
        items += ["t"] * rng.randint(1, 6)
    return items


class Kernel:
    def __init__(self, items, per_buffer: bool, rng: random.Random):
        self.items, self.per_buffer, self.rng = items, per_buffer, rng
        self.ready = [0] * KFETCH
        self.consumed = [0] * RING          # per buffer (fixed protocol)
        self.consumed_sum = 0               # one count for the ring (the racy one)
        self.p_ready = [0, 0]
        self.p_done = [0, 0]
        self.p_ready_sum = 0
        self.p_done_sum = 0
        self.desc = [None] * RING           # (kind, item index) or END
        self.slot = [[None] * KFETCH for _ in range(RING)]  # item index per fetching wave's half
        self.landed = [set() for _ in range(KFETCH)]
        self.in_flight = [[] for _ in range(KFETCH)]       # issued, not landed (in issue order)
        self.pbuf = [dict(), dict()]        # score wave -> tile index written
        self.pv_tiles = [0] * KPV           # tiles each P.V wave has finished reading

    # ---- DMA landing: in order per fetching wave, after random delays
    def land_some(self):
        for pw in range(KFETCH):
            if self.in_flight[pw] and self.rng.random() < 0.3:
                self.landed[pw].add(self.in_flight[pw].pop(0))

    def landed_through(self, pw, j):
        return all(i in self.landed[pw] for i in range(j + 1))

    # ---- roles (generators: yield when blocked)
    def fetch(self, pw):
        n = len(self.items)
        j = 0
        while True:
            if j in (2, 3):
                while not self.landed_through(pw, j - 2):
                    yield
                self.ready[pw] = max(self.ready[pw], j - 1)
            elif j > 3:
                while not self.landed_through(pw, j - 3):
                    yield
                self.ready[pw] = max(self.ready[pw], j - 2)
            if j >= RING:
                if self.per_buffer:
                    while self.consumed[j % RING] < KWAVES * (j // RING):
                        yield
                else:
                    while self.consumed_sum < KWAVES * (j - RING + 1):
                        yield
            if j >= n:
                if pw == 0:
                    self.desc[j % RING] = END
                break
            self.slot[j % RING][pw] = j
            self.in_flight[pw].append(j)
            if pw == 0:
                self.desc[j % RING] = (self.items[j], j)
            j += 1
            yield
        while self.in_flight[pw]:
            yield
        self.ready[pw] = 1 << 30

    def read_item(self, i):
        d = self.desc[i % RING]
        if d == END:
            if i != len(self.items):
                raise Violation(f"end marker read for item {i}")
            return None
        if d[1] != i:
            raise Violation(f"buffer {i % RING} holds item {d[1]}'s descriptor, item {i} expected")
        for pw in range(KFETCH):
            if self.slot[i % RING][pw] != i or i not in self.landed[pw]:
                raise Violation(f"item {i}: fetching wave {pw}'s half not in its buffer")
        return d[0]

    def consume(self, i):
        self.consumed[i % RING] += 1
        self.consumed_sum += 1

    def score(self, sw):
        i = k = 0
        while True:
            while min(self.ready) < i + 1:
                yield
            kind = self.read_item(i)
            if kind is None:
                return
            self.consume(i)
            if kind == "t":
                pb = k % 2
                if k >= 2:
                    if self.per_buffer:
                        while self.p_done[pb] < KPV * (k // 2):
                            yield
                    else:
                        while self.p_done_sum < KPV * (k - 1):
                            yield
                if any(t < k - 1 for t in self.pv_tiles):
                    raise Violation(f"score wave {sw} overwrites P buffer {pb} before tile {k - 2} was read")
                self.pbuf[pb][sw] = k
                self.p_ready[pb] += 1
                self.p_ready_sum += 1
                k += 1
            i += 1
            yield

    def pv(self, v):
        i = k = 0
        while True:
            while min(self.ready) < i + 1:
                yield
            kind = self.read_item(i)
            if kind is None:
                return
            self.consume(i)
            if kind == "t":
                pb = k % 2
                if self.per_buffer:
                    while self.p_ready[pb] < KSCORE * (k // 2 + 1):
                        yield
                else:
                    while self.p_ready_sum < KSCORE * (k + 1):
                        yield
                if any(self.pbuf[pb].get(sw) != k for sw in range(KSCORE)):
                    raise Violation(f"P.V wave {v} reads tile {k} before every score wave wrote it")
                self.p_done[pb] += 1
                self.p_done_sum += 1
                k += 1
                self.pv_tiles[v] = k
            i += 1
            yield

    def run(self, max_steps=200000):
        roles = ([self.fetch(p) for p in range(KFETCH)] + [self.score(s) for s in range(KSCORE)]
                 + [self.pv(v) for v in range(KPV)])
        # uneven speeds: each wave gets its own chance of running at a step
        speed = [self.rng.choice([0.05, 0.3, 1.0]) for _ in roles]
        live = list(range(len(roles)))
        for _ in range(max_steps):
            if not live:
                return
            self.land_some()
            for r in list(live):
                if self.rng.random() < speed[r]:
                    try:
                        next(roles[r])
                    except StopIteration:
                        live.remove(r)
        raise Violation("a schedule did not end")


@pytest.mark.parametrize("seed", range(300))
def test_per_buffer_counts_keep_every_buffer_until_read(seed):
    rng = random.Random(seed)
    Kernel(items_of(rng), per_buffer=True, rng=rng).run()


def test_ring_wide_sums_let_a_fast_wave_stand_in_for_a_slow_one():
    """The counts as sums over waves: some schedule refills a buffer, or
    overwrites or reads a P buffer, out of turn."""
    found = 0
    for seed in range(300):
        rng = random.Random(seed)
        try:
            Kernel(items_of(rng), per_buffer=False, rng=rng).run()
        except Violation:
            found += 1
    assert found > 0
