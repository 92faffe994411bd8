"""The LDS stage schedules of the forward kernels, checked on the CPU: the
64-row-wave kernel's iterations and the ping-pong kernel's slots (below).

The kernel walks a work item's keys in half-tiles of 32 through iterations of
two steps: step u runs the softmax of half-tile u, Q.K^T of half-tile u+1 and
P.V of half-tile u-1, so iteration i reads K tile i and V tile i-1. The K and V
tiles (64 keys) go through a ring of three LDS stages: tile t lives in stage
t % 3. The prologue copies K tiles 0 and 1 and V tile 0; iteration i copies K
tile i+2 and V tile i+1 (those that exist), and ends by waiting for every copy
but its own, then a workgroup barrier.

This model replays that schedule for every item length and checks what makes
it race-free: every tile an iteration reads is in its stage and its copy was
issued in an earlier iteration (so the wait and barrier that ended that
iteration made it visible), and no copy lands in a stage that the same
iteration reads or that holds a tile a later iteration still reads.
"""

import pytest

STAGES = 3


def schedule(n_half):
    """Iterations of one item with n_half half-tiles: a list of
    (reads, copies), each a list of (kind, tile, stage); plus the prologue's copies."""
    n_tiles = (n_half + 1) // 2
    prologue = [("K", 0, 0)] if n_tiles > 0 else []
    if n_tiles > 1:
        prologue.append(("K", 1, 1))
    if n_tiles > 0:
        prologue.append(("V", 0, 0))
    iters = []
    n_iter = (n_half + 1) // 2 + 1 if n_tiles > 0 else 0
    for i in range(n_iter):
        reads = []
        for u in (2 * i - 1, 2 * i):
            if 0 <= u + 1 < n_half:                       # Q.K^T of half-tile u+1
                t = (u + 1) // 2
                reads.append(("K", t, t % STAGES))
            if 1 <= u and u - 1 < n_half:                 # P.V of half-tile u-1
                t = (u - 1) // 2
                reads.append(("V", t, t % STAGES))
        copies = []
        if i + 2 < n_tiles:
            copies.append(("K", i + 2, (i + 2) % STAGES))
        if i + 1 < n_tiles:
            copies.append(("V", i + 1, (i + 1) % STAGES))
        iters.append((reads, copies))
    return prologue, iters


def check_schedule(n_half, prologue, iters):
    # when each tile becomes readable: the prologue waits for K tile 0 before
    # iteration 0 and for its other copies by the end of iteration 0; a copy
    # issued in iteration c is waited for at the end of iteration c + 1
    readable_from = {}
    for kind, t, _st in prologue:
        readable_from[(kind, t)] = 0 if (kind, t) == ("K", 0) else 1
    holder = {(kind, st): t for kind, t, st in prologue}
    last_read = {}
    for i, (reads, _) in enumerate(iters):
        for kind, t, _st in reads:
            last_read[(kind, t)] = i
    for i, (reads, copies) in enumerate(iters):
        # a copy may land as soon as it is issued: the tile its stage held must
        # not be read in this iteration or any later one
        for kind, t, st in copies:
            old = holder.get((kind, st))
            assert old is None or last_read.get((kind, old), -1) < i, (n_half, i, kind, t, old)
            holder[(kind, st)] = t
            readable_from[(kind, t)] = i + 2
        for kind, t, st in reads:
            assert holder.get((kind, st)) == t, (n_half, i, kind, t)
            assert readable_from[(kind, t)] <= i, (n_half, i, kind, t)
    # every tile's K and V are read
    for t in range((n_half + 1) // 2):
        assert ("K", t) in last_read and ("V", t) in last_read, (n_half, t)


@pytest.mark.parametrize("n_half", range(0, 41))
def test_wide_kernel_stage_ring_is_race_free(n_half):
    check_schedule(n_half, *schedule(n_half))


def test_the_model_reports_a_copy_one_tile_too_early():
    """Planted mistakes must be reported: K tile i+3 copied in iteration i lands
    in the stage K tile i is read from; with two stages instead of three, K
    tile i+2 lands where K tile i is read."""
    prologue, iters = schedule(12)
    early = [(r, [("K", i + 3, (i + 3) % STAGES)] + [c for c in cp if c[0] == "V"])
             for i, (r, cp) in enumerate(iters)]
    with pytest.raises(AssertionError):
        check_schedule(12, prologue, early)
    two = [([(k, t, t % 2) for k, t, _ in r], [(k, t, t % 2) for k, t, _ in cp])
           for r, cp in iters]
    with pytest.raises(AssertionError):
        check_schedule(12, [(k, t, t % 2) for k, t, _ in prologue], two)


# ---------------------------------------------------------------- the ping-pong kernel
#
# Two groups of waves, half a tile apart. Tile j lives in stage j % 3. Slot 2j:
# group A runs Q.K^T of tile j and P.V of tile j-1 (MFMA phase) while group B
# runs the softmax of tile j-1 and first copies K tile j+2; slot 2j+1: group B
# runs Q.K^T of tile j and P.V of tile j-1 while group A runs the softmax of
# tile j and first copies V tile j+1. A group waits for its own earlier copies
# at the end of its softmax slot (all but the ones it issued in that slot), and
# every slot ends with a workgroup barrier. The prologue copies K tiles 0 and 1
# and V tile 0 and waits for all of them; a last slot pair j = n runs the P.V
# of tile n-1.

def pingpong_schedule(n):
    """Slots of an item with n key tiles: (reads, copies, landed) per slot, where
    landed lists the copies whose wait ends this slot (visible from the next)."""
    slots = []
    pending = {"A": [], "B": []}
    for j in range(n + 1):
        for half in (0, 1):
            mfma, valu = ("A", "B") if half == 0 else ("B", "A")
            reads, copies = [], []
            if j < n:
                reads.append((mfma, "K", j, j % STAGES))
            if 1 <= j:
                reads.append((mfma, "V", j - 1, (j - 1) % STAGES))
            if half == 0 and j + 2 < n:
                copies.append((valu, "K", j + 2, (j + 2) % STAGES))
            if half == 1 and j + 1 < n:
                copies.append((valu, "V", j + 1, (j + 1) % STAGES))
            # the softmax group's wait: every copy it issued before this slot
            landed = pending[valu]
            pending[valu] = [c for c in copies if c[0] == valu]
            slots.append((reads, copies, landed))
    return slots


def check_pingpong(n, slots):
    prologue = ([("K", 0, 0), ("V", 0, 0)] if n >= 1 else []) + ([("K", 1, 1)] if n >= 2 else [])
    holder = {(k, st): t for k, t, st in prologue}
    visible = {(k, t) for k, t, _ in prologue}
    last_read = {}
    for s, (reads, _, _) in enumerate(slots):
        for _g, k, t, _st in reads:
            last_read[(k, t)] = s
    for s, (reads, copies, landed) in enumerate(slots):
        for _g, k, t, st in copies:
            old = holder.get((k, st))
            assert old is None or last_read.get((k, old), -1) < s, (n, s, k, t, old)
            holder[(k, st)] = t
        for _g, k, t, st in reads:
            assert holder.get((k, st)) == t and (k, t) in visible, (n, s, k, t)
        for _g, k, t, _st in landed:
            visible.add((k, t))


@pytest.mark.parametrize("n", range(0, 24))
def test_pingpong_stage_ring_is_race_free(n):
    check_pingpong(n, pingpong_schedule(n))


def test_pingpong_model_reports_a_late_wait():
    """Planted mistake: a group that waits for its copies one softmax slot later
    than the kernel does reads a K tile that has not landed."""
    slots = pingpong_schedule(9)
    late = [(r, c, []) for r, c, _ in slots]
    for s in range(len(slots) - 2):
        late[s + 2] = (late[s + 2][0], late[s + 2][1], late[s + 2][2] + slots[s][2])
    with pytest.raises(AssertionError):
        check_pingpong(9, late)


def test_pingpong_model_reports_a_copy_one_tile_too_early():
    """Planted mistake: K tile j+3 copied in slot 2j lands in the stage that K
    tile j is read from in that slot."""
    slots = pingpong_schedule(9)
    early = []
    for reads, copies, landed in slots:
        copies = [(g, k, t + 1, (t + 1) % STAGES) if k == "K" else (g, k, t, st)
                  for g, k, t, st in copies]
        early.append((reads, copies, landed))
    with pytest.raises(AssertionError):
        check_pingpong(9, early)
