"""Host model of the decode kernel's many-split merge protocol (CPU only).

Beyond 64 splits the decode kernel counts arrivals per group of 16 splits
and spreads the merge over the last arrivals of every group, one slice of
min(128, head_dim) output columns of one query head at a time.  This module
restates that index arithmetic (csrc/decode.hip, the tail of
decode_split_kernel) in Python and replays the protocol for every split
count the library can pick (65 .. 256), every head_dim and GQA ratio it
supports, and many arrival orders, checking that

* every output slice of a set is merged exactly once, whatever the order in
  which the splits arrive;
* the mergers are the last arrivals of their group and their count is the
  nm the merger counter waits for, so the counters are re-armed exactly once;
* a merger's global index stays below nm and nm never exceeds the split
  count, so at most 64 workgroups of a set wait at a time;
* exactly one arrival, the one that completes the last group, sees the set
  counter reach the group count, and every other merger waits for it.
"""

import random

import pytest

FAN = 16            # splits per arrival group (kDecodeFan)
SINGLE_LEVEL = 64   # splits merged by a single workgroup (kDecodeSingleLevel)
SLICE_COLS = 128    # output columns per slice merger (kSliceCols)


def merge_plan(S, G, D):
    """The kernel's constants for a set with S splits, G query heads and
    head_dim D: (NG, mpg, nm, NSL)."""
    assert S > SINGLE_LEVEL
    NG = (S + FAN - 1) // FAN
    SW = min(SLICE_COLS, D)
    NSL = G * D // SW
    gn_last = S - (NG - 1) * FAN
    mpg = min((NSL + NG - 1) // NG, FAN)
    nm = (NG - 1) * mpg + min(gn_last, mpg)
    return NG, mpg, nm, NSL


def replay(S, G, D, order):
    """Replay one launch's arrivals in `order` (a permutation of the splits).
    Returns (slices merged, merger indices, arrivals that saw the full count,
    final counter values)."""
    NG, mpg, nm, NSL = merge_plan(S, G, D)
    gcount = [0] * NG
    scount = 0
    done = 0
    merged = []
    mergers = []
    saw_all = []
    for split in order:
        grp = split // FAN
        gn = min(FAN, S - grp * FAN)
        ticket = gcount[grp]
        gcount[grp] += 1
        all_in = False
        if ticket == gn - 1:              # the group's last arrival
            gcount[grp] = 0               # re-armed for the next call
            all_in = scount == NG - 1
            scount += 1
        k = ticket - (gn - min(gn, mpg))  # merger index within the group
        if k < 0:
            continue
        if all_in:
            saw_all.append(split)
        mi = grp * mpg + k
        mergers.append(mi)
        sl = mi
        while sl < NSL:
            merged.append(sl)
            sl += nm
        done += 1
        if done == nm:                    # the last merger re-arms
            scount = 0
            done = 0
    return merged, mergers, saw_all, (gcount, scount, done)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_every_slice_merged_once(D, G):
    rng = random.Random(1000 * D + G)
    for S in range(SINGLE_LEVEL + 1, 257):
        NG, mpg, nm, NSL = merge_plan(S, G, D)
        assert 1 <= mpg <= FAN
        assert 1 <= nm <= SINGLE_LEVEL < S
        orders = [list(range(S)), list(range(S - 1, -1, -1))]
        for _ in range(3):
            o = list(range(S))
            rng.shuffle(o)
            orders.append(o)
        for order in orders:
            merged, mergers, saw_all, counters = replay(S, G, D, order)
            assert sorted(merged) == list(range(NSL)), (S, G, D)
            assert sorted(mergers) == list(range(nm)), (S, G, D)
            # exactly one arrival (the one completing the last group, always
            # a merger: it is its group's last ticket) sees the full count
            assert len(saw_all) == 1, (S, G, D)
            gcount, scount, done = counters
            assert gcount == [0] * NG and scount == 0 and done == 0, (S, G, D)


def test_mergers_are_the_last_arrivals_of_their_group():
    S, G, D = 256, 8, 256
    NG, mpg, nm, NSL = merge_plan(S, G, D)
    assert (NG, mpg, nm, NSL) == (16, 1, 16, 16)   # one 128-column slice per group finisher
    rng = random.Random(7)
    order = list(range(S))
    rng.shuffle(order)
    arrivals = {}
    for pos, split in enumerate(order):
        arrivals.setdefault(split // FAN, []).append(split)
    merged_by = {}
    gcount = [0] * NG
    for split in order:
        grp = split // FAN
        ticket = gcount[grp]
        gcount[grp] += 1
        if ticket - (FAN - mpg) >= 0:
            merged_by.setdefault(grp, []).append(split)
    for grp in range(NG):
        assert merged_by[grp] == arrivals[grp][-mpg:]


def test_small_final_group():
    # 65 splits: four full groups and a final group of one split, which then
    # holds a single merger; the slices still all get merged
    for G, D in [(1, 64), (4, 128), (8, 256), (16, 256)]:
        NG, mpg, nm, NSL = merge_plan(65, G, D)
        assert NG == 5 and nm == 4 * mpg + 1
        merged, mergers, _, _ = replay(65, G, D, list(range(65)))
        assert sorted(merged) == list(range(NSL))
