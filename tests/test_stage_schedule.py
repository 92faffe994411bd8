"""The LDS stage schedule of the 64-row-wave forward kernel, checked on the CPU.

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
