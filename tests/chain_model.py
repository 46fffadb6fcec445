"""A CPU model of the chained decode step's scheduling protocol (chain.hip).

Each wave of each workgroup is a Python generator that performs, between two
`yield`s, what the kernel's wave does between two reads of shared state: one
pass of its loop body.  A seeded random scheduler interleaves them.  The model
keeps the kernel's data structures (ticket, completion counters, the LDS ring
of slot descriptors, x-ready flags, finish counts, the two x buffers) and its
rules, and records every multiply so that the tests can check:

* every row of every slot is multiplied exactly once, with the x of its stage;
* a stage's x is staged only after every slot of the stage it depends on was
  released, and a buffer is overwritten only when no unreleased slot reads it;
* every wave finishes (no deadlock), and the control words end reset.

It is test infrastructure: nothing in the library imports it."""
import random

RING = 8          # slots a workgroup holds at once
WORKERS = 8       # worker waves per workgroup
NB = 6            # items in flight per worker
HOLD = 3          # a workgroup claims one ticket while it holds fewer slots
INF = 1 << 60


class Plan:
    """stages: list of (dep, nslots, rows_per_slot_list, nseg)."""

    def __init__(self, stages):
        self.stages = stages
        self.slots = []  # (stage, rows, nseg)
        self.slot0 = []
        for s, (dep, rows_list, nseg) in enumerate(stages):
            self.slot0.append(len(self.slots))
            for r in rows_list:
                self.slots.append((s, r, nseg))
        self.total = len(self.slots)

    def nslots(self, s):
        return len(self.stages[s][1])


class Global:
    def __init__(self, plan):
        self.ticket = 0
        self.done = [0] * len(plan.stages)
        self.exited = 0
        self.mults = {}        # (global slot, row, seg) -> count
        self.x_staged = []     # (stage, all dep slots released at that time)
        self.errors = []


class WG:
    def __init__(self):
        self.seq = [-1] * RING
        self.desc = [None] * RING   # dict(t, stage, rows, nseg, end)
        self.xready = [-1] * RING
        self.fin = [0] * RING
        self.claimed = 0
        self.released = 0
        self.q_end = INF
        self.xbuf = [None, None]    # stage held by each buffer
        self.y = [dict() for _ in range(RING)]  # row sums written by workers


def worker(g, plan, wg, w):
    ring = [None] * NB   # (q, r, seg, t, x_stage_at_issue)
    nq, nr, ns = 0, w, 0
    ended = False
    xq, xbuf_idx = -1, -1

    def issue(b):
        nonlocal nq, nr, ns, ended
        ring[b] = None
        for _ in range(RING + 1):
            if ended:
                return
            e = nq % RING
            if wg.seq[e] != nq:
                return
            d = wg.desc[e]
            if d["end"]:
                ended = True
                return
            if nr < d["rows"]:
                ring[b] = (nq, nr, ns, d["t"])
                ns += 1
                if ns == d["nseg"]:
                    ns, nr = 0, nr + WORKERS
                return
            if w >= d["rows"]:
                wg.fin[e] += 1  # no row of this slot is ours
            nq, nr, ns = nq + 1, w, 0

    for b in range(NB):
        issue(b)
    yield
    while True:
        for b in range(NB):
            it = ring[b]
            if it is not None:
                q, r, seg, t = it
                e = q % RING
                if q != xq:
                    while (wg.xready[e] >> 1) != q:
                        yield
                    xq, xbuf_idx = q, wg.xready[e] & 1
                d = wg.desc[e]
                assert d["t"] == t, "descriptor of slot %d replaced while in use" % q
                stage = plan.slots[t][0]
                if wg.xbuf[xbuf_idx] != stage:
                    g.errors.append("slot %d multiplied with x of stage %s, not %d" % (t, wg.xbuf[xbuf_idx], stage))
                g.mults[(t, r, seg)] = g.mults.get((t, r, seg), 0) + 1
                if seg == d["nseg"] - 1:
                    wg.y[e][r] = True
                    if r + WORKERS >= d["rows"]:
                        wg.fin[e] += 1
            issue(b)
            yield
        if all(x is None for x in ring):
            if ended:
                return
            yield


def stager(g, plan, wg, end_check=True):
    q_stage = 0
    last = [-1, -1]
    while True:
        if q_stage == wg.q_end:
            return
        yield  # q_end and claimed are two separate reads
        progress = False
        if q_stage < wg.claimed:
            e = q_stage % RING
            if end_check and wg.desc[e]["end"]:
                return  # past the last slot: nothing more to stage
            s = wg.desc[e]["stage"]
            if not 0 <= s < len(plan.stages):
                g.errors.append("staging slot %d of workgroup with stage %s" % (q_stage, s))
                return
            b = 0 if wg.xbuf[0] == s else 1 if wg.xbuf[1] == s else -1
            if b < 0:
                q_rel = wg.released
                fb = 0 if last[0] < q_rel else 1 if last[1] < q_rel else -1
                if fb >= 0:
                    dep = plan.stages[s][0]
                    if dep < 0 or g.done[dep] >= plan.nslots(dep):
                        if dep >= 0 and g.done[dep] != plan.nslots(dep):
                            g.errors.append("stage %d over-counted" % dep)
                        wg.xbuf[fb] = s
                        g.x_staged.append(s)
                        b = fb
            if b >= 0:
                last[b] = q_stage
                wg.xready[e] = 2 * q_stage + b
                q_stage += 1
                progress = True
        yield


def releaser(g, plan, wg, grid):
    q_claim = q_rel = 0
    q_end = INF
    while True:
        while q_rel < q_claim and q_rel != q_end:
            e = q_rel % RING
            if wg.fin[e] < WORKERS:
                break
            d = wg.desc[e]
            rows = d["rows"]
            if sorted(wg.y[e]) != list(range(rows)):
                g.errors.append("slot %d released with rows %s" % (d["t"], sorted(wg.y[e])))
            wg.y[e] = {}
            wg.fin[e] = 0
            g.done[d["stage"]] += 1
            q_rel += 1
            wg.released = q_rel
        if q_rel == q_end:
            break
        nfree = 1 if q_claim - q_rel < HOLD else 0
        if q_end == INF and nfree > 0:
            t0 = g.ticket
            g.ticket += nfree
            yield  # the atomic's round trip
            nreal = min(nfree, max(0, plan.total - t0))
            for i in range(nfree):
                e = (q_claim + i) % RING
                if i < nreal:
                    s, rows, nseg = plan.slots[t0 + i]
                    wg.desc[e] = dict(t=t0 + i, stage=s, rows=rows, nseg=nseg, end=False)
                elif i == nreal:
                    old = wg.desc[e]
                    wg.desc[e] = dict(t=-1, stage=-7 if old is None else old["stage"], rows=0, nseg=0, end=True)
            nposted = nreal + 1 if nreal < nfree else nfree
            for i in range(nposted):
                wg.seq[(q_claim + i) % RING] = q_claim + i
            if nreal < nfree:
                q_end = q_claim + nreal
            q_claim += nposted
            if q_end != INF:
                wg.q_end = q_end
                yield  # two separate writes
            wg.claimed = q_claim
        yield
    g.exited += 1
    if g.exited == grid:
        g.done = [0] * len(plan.stages)
        g.ticket = 0
        g.exited = 0


def run(plan, grid, seed, max_steps=2_000_000, end_check=True):
    """Runs one launch; returns (global state, steps, unfinished waves)."""
    rng = random.Random(seed)
    g = Global(plan)
    waves = []
    for _ in range(grid):
        wg = WG()
        for w in range(WORKERS):
            waves.append(worker(g, plan, wg, w))
        waves.append(stager(g, plan, wg, end_check))
        waves.append(releaser(g, plan, wg, grid))
    live = list(range(len(waves)))
    steps = 0
    while live and steps < max_steps:
        i = rng.randrange(len(live))
        try:
            next(waves[live[i]])
        except StopIteration:
            live[i] = live[-1]
            live.pop()
        steps += 1
    return g, steps, len(live)
