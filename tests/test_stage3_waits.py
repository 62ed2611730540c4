"""Wait counts of stage 3's c = 256 form (k3_epilogue_h256), checked on the CPU.

Each wave waits for its own direct loads with `s_waitcnt vmcnt(n)`: vector-memory
operations retire in issue order, so a wait for at most n outstanding
operations guarantees every operation issued before the last n. The functions
below restate, in Python, the order in which each kind of wave issues its
loads and stores (the kernel's prologue, loop and epilogue), and check that
at every wait the loads the following code reads are not among the last n
operations issued, for every block length the kernel meets.
"""

import pytest

NLY, NLD, NST = 8, 4, 4      # y loads per tile (waves 0-3), x loads per half tile (4-7), stores


def waves_0_3(nk):
    """Issue order of a wave of waves 0-3 over a block of nk 64-pair tiles, with
    the waits: ('L', tag) loads, ('S', h) stores, ('W', n, tag) = wait vmcnt(n),
    after which the loads of `tag` must be complete."""
    nh = 2 * nk
    ops = [("L", ("y", 0))] * NLY
    ops.append(("W", 0, ("y", 0)))                        # the prologue's transpose of half 0
    for h in range(nh):
        if h + 1 < nh and h % 2 == 1:
            ops.append(("W", NST, ("y", (h + 1) // 2)))  # the first half of the next tile
        if h % 2 == 0 and h // 2 + 1 < nk:
            ops += [("L", ("y", h // 2 + 1))] * NLY       # between the MFMAs of phase 1
        ops += [("S", h - 1)] * NST                       # phase 2
    ops += [("S", nh - 1)] * NST
    return ops


def waves_4_7(nk):
    nh = 2 * nk
    ops = [("L", ("x", 0))] * NLD
    ops.append(("W", 0, ("x", 0)))
    ops += [("L", ("x", 1))] * NLD
    for h in range(nh):
        if h + 1 < nh:
            ops.append(("W", 0, ("x", h + 1)))
            if h + 2 < nh:
                ops += [("L", ("x", h + 2))] * NLD
    return ops


def check(ops):
    issued = []
    for op in ops:
        if op[0] == "W":
            _, n, tag = op
            done = issued[: len(issued) - n] if n else issued
            pending = issued[len(done):]
            assert ("L", tag) in issued, ("waits for loads never issued", tag)
            assert ("L", tag) not in pending, ("a wait leaves needed loads in flight", tag, n)
        else:
            issued.append(op)
    return issued


@pytest.mark.parametrize("nk", range(1, 9))
def test_every_wait_covers_the_loads_it_guards(nk):
    for fn in (waves_0_3, waves_4_7):
        check(fn(nk))


@pytest.mark.parametrize("nk", range(1, 9))
def test_every_tile_is_loaded_and_every_half_tile_stored_once(nk):
    nh = 2 * nk
    ops0 = check(waves_0_3(nk))
    assert sorted({t for k, t in ops0 if k == "L"}) == [("y", t) for t in range(nk)]
    stores = [h for k, h in ops0 if k == "S"]
    assert sorted(h for h in set(stores) if h >= 0) == list(range(nh))
    assert all(stores.count(h) == NST for h in range(nh))
    ops1 = check(waves_4_7(nk))
    assert sorted({t for k, t in ops1 if k == "L"}) == [("x", h) for h in range(nh)]


def test_a_wait_one_short_is_caught():
    # the check fails if a wait allowed one more operation in flight than the
    # stores issued after the loads it guards
    ops = waves_0_3(3)
    bad = [("W", NST + 1, op[2]) if op[0] == "W" and op[1] == NST else op for op in ops]
    with pytest.raises(AssertionError):
        check(bad)
