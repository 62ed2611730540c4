"""Hand-set wait counts of the kernels' direct loads, checked on the CPU.

A wave waits for its own direct loads with `s_waitcnt vmcnt(n)`: vector-memory
operations retire in issue order, so a wait for at most n outstanding
operations guarantees every operation issued before the last n. The functions
below restate, in Python, the order in which each kind of wave issues its
loads and stores (prologue, loop and epilogue) in the three kernels that set
such counts by hand -- stage 1 at c_z = 256 (k1_ln_proj_wide), stage 2
(k2_contract_p and the 128 x 128 tile) and stage 3 at c = 256
(k3_epilogue_h256) -- and check that at every wait the loads the following
code reads are not among the last n operations issued, for every block length
the kernels meet. (The other kernels load into registers and leave the counts
to the compiler.)
"""

import pytest

# ---- stage 3, c = 256 ----
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


# ---- stage 1, c_z = 256 (k1_ln_proj_wide): every wave ----
K1_NLD, K1_STORES = 4, 8     # x loads per tile, plane stores per tile step (2 per pair group)


def stage1_wide(nk):
    """('L', tag): the mask load of a tile ('m', step) or its x loads ('x', step)"""
    ops = [("L", ("m", 0))] + [("L", ("x", 0))] * K1_NLD + [("L", ("x", 1))] * K1_NLD
    ops += [("S", -1)] * K1_STORES                       # stand-ins past the end of the plane
    ops.append(("W", K1_NLD + K1_STORES, ("x", 0)))      # tile 0's rows, before its LayerNorm
    ops.append(("W", K1_NLD + K1_STORES, ("m", 0)))
    for k in range(nk):
        ops += [("L", ("m", k + 1))] + [("L", ("x", k + 2))] * K1_NLD
        ops.append(("W", K1_STORES + 1 + K1_NLD, ("x", k + 1)))   # tile k + 1's rows, before its LayerNorm
        ops += [("S", k)] * K1_STORES                    # the gates' plane stores, 2 per group step
    return ops


# ---- stage 2 (k2_contract_p, the persistent 256 x 256 tile): every wave ----
K2_PER_STEP, K2_STORES = 8, 16   # direct loads per k-step, y stores per tile


def stage2_persistent(count, nk):
    """count tiles of nk k-steps; ('L', (tile, step)) fills"""
    ops = [("L", (0, 0))] * K2_PER_STEP
    for k in range(count):
        for kt in range(nk):
            ops.append(("W", K2_STORES if kt == 0 and k > 0 else 0, (k, kt)))
            if kt + 1 < nk:
                ops += [("L", (k, kt + 1))] * K2_PER_STEP
        if k + 1 < count:
            ops += [("L", (k + 1, 0))] * K2_PER_STEP     # the next tile's first fill, before the epilogue
        ops += [("S", k)] * K2_STORES
    return ops


# ---- stage 2, the 128 x 128 tile (three ring stages, one tile per block) ----
K2S_PER_STEP = 4


def stage2_small(nk):
    ops = []
    for s in range(2):
        if s < nk:
            ops += [("L", s)] * K2S_PER_STEP
    for kt in range(nk):
        later = min(1, nk - 1 - kt)
        ops.append(("W", K2S_PER_STEP * later, kt))
        if kt + 2 < nk:
            ops += [("L", kt + 2)] * K2S_PER_STEP
    return ops


@pytest.mark.parametrize("nk", range(1, 10))
def test_stage1_wide_waits(nk):
    check(stage1_wide(nk))


@pytest.mark.parametrize("count", range(1, 6))
@pytest.mark.parametrize("nk", [1, 2, 3, 12, 24])
def test_stage2_persistent_waits(count, nk):
    check(stage2_persistent(count, nk))


@pytest.mark.parametrize("nk", range(1, 6))
def test_stage2_small_tile_waits(nk):
    check(stage2_small(nk))


def test_stage1_and_stage2_waits_one_short_are_caught():
    for ops in (stage1_wide(3), stage2_persistent(3, 4)):
        bad = [("W", op[1] + 1, op[2]) if op[0] == "W" and op[1] > 0 else op for op in ops]
        with pytest.raises(AssertionError):
            check(bad)
