"""Host model of the MLA kernel's shared merge protocol, under random interleavings.

The kernel's split pieces of a unit publish partials, add one to the unit's
arrival counter (low 16 bits), and after their stream:
  - wait, polling a bounded number of times, until every piece has arrived
    (the last arriver does not wait),
  - claim slice "split index" (if < nsl) with an atomic OR on the claim mask,
    merge it, then claim and merge any slice still free until none is left,
  - leave (add 2^16); the last to leave clears the counter and the mask.
This model runs those steps as atomic actions in random orders, with pieces
that stop waiting at random, and checks: every slice is merged exactly once,
only after every piece has arrived; the counter and mask end at zero; and no
piece touches the unit's words after the reset.  A planted mistake (the last
arriver not sweeping) must be caught.
"""
import random

import pytest

ARRIVE_MASK, LEAVE = 0xFFFF, 1 << 16


def simulate(ns, nsl, rng, give_up_p=0.3, last_sweeps=True):
    st = {"cnt": 0, "claim": 0, "merged": [0] * nsl, "reset": False, "arrivals_at_merge": []}
    # each piece is a generator of atomic steps
    def piece(s):
        yield
        old = st["cnt"]
        st["cnt"] += 1                      # arrival
        last = (old & ARRIVE_MASK) == ns - 1
        yield
        ready = last
        polls = 0
        while not ready:
            if rng.random() < give_up_p / 4:  # this piece stops polling
                break
            ready = (st["cnt"] & ARRIVE_MASK) == ns
            polls += 1
            yield
        if ready:
            want = s if s < nsl else None
            seen = 0
            while True:
                assert not st["reset"]
                if want is None:
                    free = ((1 << nsl) - 1) & ~seen
                    if free == 0 or (not last_sweeps and last):
                        break
                    want = (free & -free).bit_length() - 1
                bit = 1 << want
                old_c = st["claim"]
                st["claim"] |= bit                   # atomic OR
                seen |= old_c | bit
                got = not (old_c & bit)
                if got:
                    st["merged"][want] += 1
                    st["arrivals_at_merge"].append(st["cnt"] & ARRIVE_MASK)
                want = None
                yield
        assert not st["reset"]
        old = st["cnt"]
        st["cnt"] += LEAVE                           # leave
        if (old >> 16) == ns - 1:
            st["cnt"] = 0
            st["claim"] = 0
            st["reset"] = True
        yield

    gens = [piece(s) for s in range(ns)]
    live = list(range(ns))
    while live:
        i = rng.choice(live)
        try:
            next(gens[i])
        except StopIteration:
            live.remove(i)
    return st


@pytest.mark.parametrize("seed", range(200))
def test_every_slice_merged_once_and_words_cleared(seed):
    rng = random.Random(seed)
    ns = rng.choice([2, 3, 5, 9, 16, 17, 31])
    nsl = min(ns, 16)
    st = simulate(ns, nsl, rng, give_up_p=rng.choice([0.0, 0.3, 1.0]))
    assert st["merged"] == [1] * nsl
    assert all(a == ns for a in st["arrivals_at_merge"])
    assert st["reset"] and st["cnt"] == 0 and st["claim"] == 0


def test_planted_mistake_last_arriver_without_sweep_is_caught():
    """Without the last arriver's sweep, a slice whose piece stopped waiting is
    never merged on some interleavings."""
    missed = 0
    for seed in range(200):
        rng = random.Random(seed)
        st = simulate(9, 9, rng, give_up_p=1.0, last_sweeps=False)
        missed += st["merged"] != [1] * 9
    assert missed > 0
