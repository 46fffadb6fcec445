"""The chained decode step's scheduling protocol, checked on the CPU.

tests/chain_model.py models every wave of every workgroup of chain.hip as a
step machine (one pass of the wave's loop per step, shared words read and
written as the kernel does, with the kernel's ring sizes) under seeded random
interleavings.  For several plans and grids these tests check that every
interleaving tried finishes (no deadlock), multiplies every row of every slot
exactly once with the x of its own stage, stages x only after its producing
stage was released everywhere, and leaves the control words reset.  A planted
mistake (the staging wave without its END-entry check, the race that let it
read a stale descriptor) must be caught, which shows the model exercises the
interleavings that matter.  Page: "1-bit quantization is not magic", section
3.3 (launch overhead: the steps of a decode layer fused into one launch)."""
import random

import pytest

import chain_model as cm


def layer_plan(layers, nslots=(6, 2, 10, 2), rows=(24, 8, 48, 8), nseg=(1, 1, 1, 3)):
    st = []
    for _ in range(layers):
        for j in range(4):
            st.append((len(st) - 1 if st else -1, [rows[j]] * nslots[j], nseg[j]))
    return cm.Plan(st)


def ragged_plan(seed):
    g = random.Random(seed)
    st = []
    for s in range(g.randint(3, 9)):
        dep = g.randint(-1, s - 1) if s else -1
        n = g.randint(1, 12)
        st.append((dep, [g.choice([8, 16, 24, 64, 1, 3, 57]) for _ in range(n)], g.randint(1, 4)))
    return cm.Plan(st)


def check(plan, g, live):
    assert live == 0, "waves left unfinished (deadlock)"
    assert not g.errors, g.errors[:3]
    want = {(t, r, seg) for t, (s, rows, nseg) in enumerate(plan.slots) for r in range(rows) for seg in range(nseg)}
    assert set(g.mults) == want, "rows missed or invented"
    assert all(c == 1 for c in g.mults.values()), "a row multiplied twice"
    assert g.ticket == 0 and g.exited == 0 and not any(g.done), "control words not reset"


@pytest.mark.parametrize("grid", [1, 3, 7])
@pytest.mark.parametrize("seed", range(6))
def test_layers(grid, seed):
    plan = layer_plan(2)
    g, steps, live = cm.run(plan, grid, seed)
    check(plan, g, live)


@pytest.mark.parametrize("seed", range(12))
def test_ragged_plans(seed):
    plan = ragged_plan(seed)
    g, steps, live = cm.run(plan, 1 + seed % 5, seed)
    check(plan, g, live)


def test_more_workgroups_than_slots():
    plan = cm.Plan([(-1, [8, 8], 1), (0, [8], 2)])
    for seed in range(10):
        g, steps, live = cm.run(plan, 6, seed)
        check(plan, g, live)


def test_planted_end_race_is_caught():
    plan = layer_plan(2)
    failures = 0
    for seed in range(40):
        g, steps, live = cm.run(plan, 5, seed, end_check=False)
        failures += bool(g.errors or live)
    assert failures > 0
