"""The split-K tile-state protocol of the LDS tile, checked as a model on the
CPU.  Each output tile has three 32-bit words: word 0 counts arrivals over all
launches (each launch adds exactly 8), words 1 and 2 hold the slice claims of
even and odd epochs.  In a launch with S splits (S = 2, 4 or 8):

- every split adds 1 to word 0 once its partials are stored; the one that gets
  back rank S - 1 is the last, adds 8 - S more and clears the claim word of
  the next epoch;
- with S >= 4 a split that is not last may wait, bounded, until word 0 shows
  all S arrivals; if it saw them it claims its own slice with an atomic OR on
  the epoch's claim word and adds the slice if the bit was still clear;
- the last adds its own slice, then claims every other slice with one atomic
  OR and adds those whose bits were still clear.

The model runs each workgroup as a sequence of atomic steps, interleaves them
at random, lets waits give up at random, and checks that every slice of every
launch is added exactly once, that word 0 is a multiple of 8 between launches
and that no reset is ever needed, across launches of mixed S and across the
wrap of word 0 at 2**32."""
import random

import pytest

MASK = 0xFFFFFFFF


class Tile:
    def __init__(self, w0=0):
        self.w = [w0 & MASK, 0, 0]

    def fetch_add(self, i, v):
        old = self.w[i]
        self.w[i] = (old + v) & MASK
        return old

    def fetch_or(self, i, v):
        old = self.w[i]
        self.w[i] = old | v
        return old


def workgroup(tile, S, split, added, rng, may_wait, clear=True):
    """One split's steps; each `yield` is a point where others may run.
    clear=False plants a mistake: the last arrival leaves the next epoch's
    claim word as it is."""
    old = tile.fetch_add(0, 1)
    yield
    last = (old & 7) == S - 1
    epoch_word = 1 + ((old >> 3) & 1)
    if last:
        if S < 8:
            tile.fetch_add(0, 8 - S)
            yield
        if clear:
            tile.w[1 + (((old >> 3) + 1) & 1)] = 0
        yield
    if S < 4:
        if last:
            added.extend(range(S))          # the whole tile (one slice per split, all added here)
        return
    if last:
        added.append(split)
        yield
        others = ((1 << S) - 1) & ~(1 << split)
        got = others & ~tile.fetch_or(epoch_word, others)
        yield
        added.extend(sl for sl in range(S) if (got >> sl) & 1)
        return
    ready = False
    if may_wait:
        base = old & ~7 & MASK
        while True:
            ready = ((tile.w[0] - base) & MASK) >= S
            if ready or rng.random() < 0.05:    # the bounded wait may run out
                break
            yield
    if ready:
        bit = 1 << split
        if not tile.fetch_or(epoch_word, bit) & bit:
            yield
            added.append(split)


def run_launch(tile, S, rng, may_wait, clear=True):
    added = []
    gens = [workgroup(tile, S, s, added, rng, may_wait, clear) for s in range(S)]
    # workgroups start in any order and at any time
    live = list(gens)
    rng.shuffle(live)
    while live:
        g = rng.choice(live)
        try:
            next(g)
        except StopIteration:
            live.remove(g)
    return added


@pytest.mark.parametrize("start", [0, MASK - 8 * 37 + 1])
def test_every_slice_added_once_without_reset(start):
    rng = random.Random(1234 + start)
    tile = Tile(start)
    for launch in range(3000):
        S = rng.choice((2, 4, 8))
        assert tile.w[0] % 8 == 0
        before = tile.w[0]
        added = run_launch(tile, S, rng, may_wait=rng.random() < 0.8)
        assert sorted(added) == list(range(S)), (launch, S, added)
        assert tile.w[0] == (before + 8) & MASK
        # the claim word the next launch uses is clear when it starts
        assert tile.w[1 + ((tile.w[0] >> 3) & 1)] == 0


def test_waits_off_leave_every_slice_to_the_last():
    rng = random.Random(7)
    tile = Tile()
    for _ in range(500):
        S = rng.choice((4, 8))
        assert sorted(run_launch(tile, S, rng, may_wait=False)) == list(range(S))


def test_a_planted_missing_clear_is_caught():
    """Without the last arrival's clearing of the next epoch's claim word, a
    launch finds the claims of the launch two before it and loses slices: the
    exactly-once check fails, which shows that it can."""
    rng = random.Random(3)
    tile = Tile()
    lost = False
    for _ in range(200):
        S = rng.choice((4, 8))
        if sorted(run_launch(tile, S, rng, may_wait=True, clear=False)) != list(range(S)):
            lost = True
            break
    assert lost
