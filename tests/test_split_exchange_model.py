"""CPU model of the row-sum exchange between the two workgroups of the chunked prefill's
split carry (kda_carry.hip, carry_split_kernel), checked over random and adversarial
interleavings of the two halves.

Each half runs, per chunk c, in the kernel's order:
  - at the chunk's start: publish chunk c-1's sums into its own slot (c-1) % SLOTS, tagged c;
  - mid-chunk: check the words it loaded for the other half's chunk c-2 (expected tag c-1),
    and while the tag is not there, load the slot again;
  - at the chunk's end: load the other half's slot (c-1) % SLOTS for the next check.
After the last chunk: publish it, check the chunk before, then load and check the last one.
A load may return anywhere between its issue and the next step that uses it (the model
returns the value current when the half next moves).  The properties: every check ends
with the tag it expects (no slot was overwritten before it was read), and no schedule
deadlocks.  With 2 slots instead of 4 the overwrite becomes reachable, which the test
also shows, so the model can tell the two apart."""
import random

import pytest


def _program(n):
    """The sequence of steps of one half over n chunks."""
    steps = []
    for c in range(n):
        if c >= 1:
            steps.append(("publish", c - 1))
        if c >= 2:
            steps.append(("check", c - 2))
        steps.append(("load", max(c - 1, 0)))  # for the next chunk's check
    steps.append(("publish", n - 1))
    if n >= 2:
        steps.append(("check", n - 2))
    steps.append(("load", n - 1))
    steps.append(("check", n - 1))
    return steps


def _simulate(n, slots, rng, bias):
    """Run both halves to completion under a random schedule (half 0 is picked with
    probability `bias`); returns None, or a description of a violated property."""
    mem = [[0] * slots for _ in range(2)]  # mem[half][slot] = tag (0: nothing)
    prog = [_program(n), _program(n)]
    pc = [0, 0]
    pending = [None, None]   # (slot) of an issued load not yet returned
    loaded = [None, None]    # the tag the last load returned
    while pc[0] < len(prog[0]) or pc[1] < len(prog[1]):
        ready = [h for h in (0, 1) if pc[h] < len(prog[h])]
        h = ready[0] if len(ready) == 1 else (0 if rng.random() < bias else 1)
        other = 1 - h
        if pending[h] is not None:  # the load returns now, with the value current now
            loaded[h] = mem[other][pending[h]]
            pending[h] = None
        kind, chunk = prog[h][pc[h]]
        if kind == "publish":
            mem[h][chunk % slots] = chunk + 1
            pc[h] += 1
        elif kind == "load":
            pending[h] = chunk % slots
            pc[h] += 1
        else:  # check: the tag must be chunk + 1; a newer one means the slot was overwritten
            tag = loaded[h]
            if tag == chunk + 1:
                pc[h] += 1
            elif tag is not None and tag > chunk + 1:
                return f"half {h} read tag {tag} for chunk {chunk}: the slot was overwritten"
            else:
                # not there yet: poll again (only if the other half can still move, else deadlock)
                if pc[other] >= len(prog[other]) and mem[other][chunk % slots] != chunk + 1:
                    return f"half {h} waits for chunk {chunk} after the other half ended"
                pending[h] = chunk % slots
                if pc[other] >= len(prog[other]):
                    loaded[h] = mem[other][pending[h]]
                    pending[h] = None
    return None


@pytest.mark.parametrize("n", [1, 2, 3, 5, 9])
def test_four_slots_hold_under_random_schedules(n):
    rng = random.Random(1234 + n)
    for trial in range(3000):
        bias = (0.02, 0.2, 0.5, 0.8, 0.98)[trial % 5]
        err = _simulate(n, 4, rng, bias)
        assert err is None, (n, trial, err)


def test_two_slots_can_be_overwritten():
    """The model finds the overwrite the four slots prevent: with two, a half that runs far
    enough ahead rewrites a slot before the other half has read it."""
    rng = random.Random(7)
    found = any(_simulate(9, 2, rng, bias) for bias in (0.02, 0.98) for _ in range(2000))
    assert found
