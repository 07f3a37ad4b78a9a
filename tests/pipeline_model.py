"""A model of the kernels' LDS buffer schedules, for hazard checks on the CPU.

Each kernel runs two groups of four waves that meet at workgroup barriers;
between two barriers (an "interval") a group issues global -> LDS copies
into its buffers, reads buffers, and may wait for its own copies.  The
functions below list, per group and interval, what the kernel's loop does,
in the loop's own order; `check` then replays them:
  * a copy issued in interval i may land at any time from i on, so no group
    may read that buffer's previous tile in interval i or later;
  * a read of tile x from buffer b in interval i needs x's copy to have been
    waited for by its issuing group in an interval before i (the barrier
    between then publishes it to every wave);
  * a read marked unused (its result is thrown away) may see anything;
  * a group's overwrite of a buffer (output staging) in interval i destroys
    its tile from i on.
A wait either drains all of the group's copies or all but those issued in
the current interval (vmcnt counts in issue order).

Test infrastructure; it imports nothing from the product.
"""

from dataclasses import dataclass, field


@dataclass
class Interval:
    copies: list = field(default_factory=list)   # (buffer, tile)
    clobbers: list = field(default_factory=list)  # buffers overwritten with a group's own data
    reads: list = field(default_factory=list)    # (buffer, tile or None for unused)
    wait: str = ""                               # "", "all", "keep_current"


class Group:
    """Builds a group's intervals; barrier() closes the current one."""

    def __init__(self):
        self.intervals = [Interval()]

    @property
    def cur(self):
        return self.intervals[-1]

    def copy(self, buf, tile):
        self.cur.copies.append((buf, tile))

    def read(self, buf, tile):
        self.cur.reads.append((buf, tile))

    def clobber(self, buf):
        self.cur.clobbers.append(buf)

    def wait(self, kind="all"):
        self.cur.wait = kind

    def barrier(self):
        self.intervals.append(Interval())


def check(groups):
    """Replays the groups' intervals; returns a list of hazard messages
    (empty when the schedule is safe)."""
    n = len(groups[0].intervals)
    if any(len(g.intervals) != n for g in groups):
        return ["groups pass different numbers of barriers: %s" % [len(g.intervals) for g in groups]]
    content = {}     # buffer -> tile it holds (once the last copy lands)
    issued = {}      # buffer -> interval of the last copy into it
    ready = {}       # buffer -> interval after which its last copy is published
    pending = [[] for _ in groups]   # per group: buffers with copies not yet waited for
    problems = []
    for i in range(n):
        # Copies issued in this interval (they may land at any point in it).
        for gi, g in enumerate(groups):
            for buf, tile in g.intervals[i].copies:
                content[buf] = tile
                issued[buf] = i
                ready.pop(buf, None)
                pending[gi].append((buf, i))
            for buf in g.intervals[i].clobbers:
                content[buf] = ("staged", gi)
                issued[buf] = i
                ready.pop(buf, None)
        for gi, g in enumerate(groups):
            for buf, tile in g.intervals[i].reads:
                if tile is None:
                    continue
                if content.get(buf) != tile:
                    problems.append("interval %d: group %d reads tile %s from buffer %s, which holds %s"
                                    % (i, gi, tile, buf, content.get(buf)))
                elif buf not in ready or ready[buf] >= i:
                    problems.append("interval %d: group %d reads buffer %s (tile %s) before its copy (issued in "
                                    "interval %s) is waited for and published" % (i, gi, buf, tile, issued.get(buf)))
        # Waits at the end of the interval.
        for gi, g in enumerate(groups):
            kind = g.intervals[i].wait
            if not kind:
                continue
            keep = [(b, j) for (b, j) in pending[gi] if kind == "keep_current" and j == i]
            for b, j in pending[gi]:
                if (b, j) not in keep and issued.get(b) == j:
                    ready[b] = i
            pending[gi] = keep
    return problems


# ---------------------------------------------------------------------------
# Forward (bf16 and FP8): K tiles copied by group 0 into K0..K2, V tiles by
# group 1 into V0..V2; tile t in buffer t % 3.  Step t's matrix phase reads
# V(t) (O += P V) and K(t + 1) (S of the next tile; on the last step that
# read is of a stale buffer and unused); its vector phase is the softmax of
# tile t + 1, and (bf16, d = 128) reads the first operands of V(t + 1) for
# the next matrix phase.  Group 1 runs one interval behind group 0.
#
# The kernels copy tiles 0 and 1 before the first barrier and tile 2 right
# after it (once both groups' first score products are issued); then, at the
# start of its vector phase of step t, each group copies tile t + 3 into the
# buffer of tile t and waits for everything but that copy at the phase's end.
# `ahead` = 2 with copy_at = "matrix" is the earlier schedule (tile t + 2
# copied at the start of the matrix phase, all copies waited for at the end
# of the vector phase).  Under the causal mask a bf16 wave skips the
# products and softmax of the tiles past its last query but keeps every
# copy, wait and barrier; dropping reads adds no hazard, so the model keeps
# them all.
# ---------------------------------------------------------------------------
def forward_schedule(num_kt, preload_v, ahead=3, copy_at="vector", bufs=3, waits=True):
    groups = [Group(), Group()]
    tensor = ("K", "V")
    for gi, g in enumerate(groups):
        def copy(t):
            if t < num_kt:
                g.copy("%s%d" % (tensor[gi], t % bufs), (tensor[gi], t))
                return True
            return False
        for t in range(min(2, num_kt)):
            copy(t)
        g.wait("all")
        g.barrier()
        if num_kt > 0:
            g.read("K0", ("K", 0))                     # S of tile 0
        if ahead == 3:
            copy(2)
        if preload_v and num_kt > 0:
            g.read("V0", ("V", 0))
        if gi == 1:
            g.barrier()
        for t in range(num_kt):
            copied = False
            if copy_at == "matrix":
                copied = copy(t + ahead)
            g.read("V%d" % (t % bufs), ("V", t))
            g.read("K%d" % ((t + 1) % bufs), ("K", t + 1) if t + 1 < num_kt else None)
            g.barrier()
            if copy_at == "vector":
                copied = copy(t + ahead)
            if preload_v and t + 1 < num_kt:
                g.read("V%d" % ((t + 1) % bufs), ("V", t + 1))
            if waits:
                g.wait("keep_current" if copied and copy_at == "vector" else "all")
            g.barrier()
        if gi == 0:
            g.barrier()
    return groups


# ---------------------------------------------------------------------------
# FP8 forward with three groups (12 waves, one wave of each group per SIMD):
# a step is a matrix phase (P V of tile t with V(t), the scores of tile t + 1
# with K(t + 1)) and the softmax in two halves, each phase ending at a
# barrier; group g runs g intervals behind group 0, so at any time one group
# of each SIMD is in its matrix phase and two in their exponentials.  Group 0
# copies K tile t + 3 (buffer t % 3) and group 1 V tile t + 2 (buffer
# (t + 2) % 3) at the start of the first softmax half of step t, each waiting
# at that half's end for all its copies but that one.  Tiles 0-2 of K and 0-1
# of V are copied before the first barrier.  After the loop group g passes
# 2 - g more barriers, then every wave stages its output rows from the start
# of the LDS (`stage` lists the buffers each group's rows cover).
# ---------------------------------------------------------------------------
def fp8_three_group_schedule(num_kt, bufs=3, k_ahead=3, v_ahead=2, stage=(("K0", "K1", "K2", "V0"), ("V1", "V2"), ())):
    groups = [Group(), Group(), Group()]
    for gi, g in enumerate(groups):
        def copy(tensor, t):
            if t < num_kt:
                g.copy("%s%d" % (tensor, t % bufs), (tensor, t))
                return True
            return False
        if gi == 0:
            for t in range(min(k_ahead, num_kt)):
                copy("K", t)
        if gi == 1:
            for t in range(min(v_ahead, num_kt)):
                copy("V", t)
        g.wait("all")
        g.barrier()
        if num_kt > 0:
            g.read("K0", ("K", 0))                     # S of tile 0
        for _ in range(gi):
            g.barrier()
        for t in range(num_kt):
            g.read("V%d" % (t % bufs), ("V", t))
            if t + 1 < num_kt:
                g.read("K%d" % ((t + 1) % bufs), ("K", t + 1))
            g.barrier()
            if gi in (0, 1):
                copied = copy("K", t + k_ahead) if gi == 0 else copy("V", t + v_ahead)
                g.wait("keep_current" if copied else "all")
            g.barrier()
            g.barrier()
        for _ in range(2 - gi):
            g.barrier()
        for buf in stage[gi]:
            g.clobber(buf)
    return groups


# ---------------------------------------------------------------------------
# Backward dK/dV kernel: group g walks its steps r (blocks 2 r + g of the
# visited list) in its own two buffers, step r in buffer r % 2.  Matrix
# phase of round r: the gradient products of step r - 1 and the score
# products of step r (with the row terms of step r as the accumulators'
# start values).  Vector phase: the copy of step r + 1 into buffer
# (r + 1) % 2, P and dS of step r (from registers), wait for all.
# A wave runs no products for steps its group does not have, nor for the
# causal steps whose queries all come before its keys, nor the gradient
# products of round 0 or the score products past its last step; it still
# issues its share of every copy and passes every wait and barrier, so the
# model (which keeps every read) covers it.
# ---------------------------------------------------------------------------
def dkdv_schedule(n_blk, bufs=2, copy_in_vector=True):
    R = (n_blk + 1) // 2
    groups = [Group(), Group()]
    for g_i, g in enumerate(groups):
        def has(r):
            return r >= 0 and 2 * r + g_i < n_blk

        def buf(r):
            return "g%d.%d" % (g_i, r % bufs)
        if has(0):
            g.copy(buf(0), (g_i, 0))
        g.wait("all")
        g.barrier()
        if g_i == 1:
            g.barrier()
        for r in range(R + 1):
            g.read(buf(r - 1), (g_i, r - 1) if has(r - 1) else None)
            g.read(buf(r), (g_i, r) if has(r) else None)
            if not copy_in_vector and has(r + 1):
                g.copy(buf(r + 1), (g_i, r + 1))
            g.barrier()
            if copy_in_vector and has(r + 1):
                g.copy(buf(r + 1), (g_i, r + 1))
            g.wait("all")
            g.barrier()
        if g_i == 0:
            g.barrier()
    return groups


# ---------------------------------------------------------------------------
# Backward dQ kernel: three buffers per group, step r in buffer r % 3,
# steps 0 and 1 copied before the loop (as above, a wave skips the products
# of steps it has no key of, never a copy, wait or barrier).  Vector phase of round r: the copy
# of step r + 2 into buffer (r + 2) % 3 (that of step r - 1), then a wait
# that leaves only that copy in flight (or drains all when none was issued).
# ---------------------------------------------------------------------------
def dq_schedule(n_blk, bufs=3, ahead=2):
    R = (n_blk + 1) // 2
    groups = [Group(), Group()]
    for g_i, g in enumerate(groups):
        def has(r):
            return r >= 0 and 2 * r + g_i < n_blk

        def buf(r):
            return "g%d.%d" % (g_i, r % bufs)
        for r in range(ahead):
            if has(r):
                g.copy(buf(r), (g_i, r))
        g.wait("all")
        g.barrier()
        if g_i == 1:
            g.barrier()
        for r in range(R + 1):
            g.read(buf(r - 1), (g_i, r - 1) if has(r - 1) else None)
            g.read(buf(r), (g_i, r) if has(r) else None)
            g.barrier()
            issued = has(r + ahead)
            if issued:
                g.copy(buf(r + ahead), (g_i, r + ahead))
            g.wait("keep_current" if issued else "all")
            g.barrier()
        if g_i == 0:
            g.barrier()
    return groups
