"""Host-side model of the fused backward's ordered dQ accumulation.

The fused backward kernel runs one workgroup per (sequence, KV head, 128-key
block).  Each workgroup walks the 64-row query tiles its keys can see (times
the query heads of its GQA group) and adds its partial dQ of every tile into
an fp32 accumulator, in a fixed order: for each tile, the key blocks that
contribute to it take turns in DESCENDING block order, each waiting until a
per-tile counter equals the number of contributors above it.  Work items are
handed out from per-XCD queues in the same descending block order.

This module restates, independently of the kernel source, (1) which key
blocks contribute to which query tile (brute force from the mask definition
and the closed form the kernel uses) and (2) a discrete-event simulation of
the queues, resident workgroups and turn waits.  The simulation is used by
tests/test_dq_order.py to show that the waits cannot deadlock for any number
of resident workgroups per XCD, and by hand to compare pipeline choices.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field

BN = 128   # keys per work item (4 waves x 32 keys)
BQ = 64    # query rows per step
NXCD = 8


def block_tiles(lq, lk, wl, wr, n):
    """Query tiles [mb_begin, mb_end) that key block n walks (the kernel's
    per-item bounds: queries that can see any key of the block)."""
    n0 = BN * n
    if n0 >= lk or lq == 0:
        return 0, 0
    off = lk - lq
    klast = min(n0 + BN - 1, lk - 1)
    i_lo = max(0, n0 - wr - off) if wr >= 0 else 0
    i_hi = min(lq, klast + wl - off + 1) if wl >= 0 else lq
    mb_begin = i_lo // BQ
    mb_end = -(-i_hi // BQ) if i_hi > i_lo else mb_begin
    return mb_begin, mb_end


def contributors_brute(lq, lk, wl, wr):
    """tile -> sorted list of key blocks whose walk includes it."""
    nblk = -(-lk // BN)
    out = {m: [] for m in range(-(-lq // BQ))}
    for n in range(nblk):
        b, e = block_tiles(lq, lk, wl, wr, n)
        for m in range(b, e):
            out[m].append(n)
    return out


def contributors_closed(lq, lk, wl, wr, m):
    """[n_lo, n_hi] of the key blocks contributing to tile m (empty if
    n_lo > n_hi): block n reaches tile m iff 128 n < 64 m + 64 + wr + off
    (its first visible query is in or before the tile) and
    128 n + 128 + wl - off > 64 m (its last visible query is in or after it).
    Floor division of possibly negative numerators."""
    off = lk - lq
    nblk = -(-lk // BN)
    n_hi = nblk - 1
    if wr >= 0:
        n_hi = min(n_hi, (BQ * m + BQ - 1 + wr + off) // BN)
    n_lo = 0
    if wl >= 0:
        n_lo = max(0, (BQ * m - wl + off) // BN)
    return n_lo, n_hi


def pairs_actual(lq, lk, wl, wr):
    """Allowed (query, key) pairs, bottom-right aligned window."""
    off = lk - lq
    total = 0
    for i in range(lq):
        lo = 0 if wl < 0 else max(0, i + off - wl)
        hi = lk - 1 if wr < 0 else min(lk - 1, i + off + wr)
        total += max(0, hi - lo + 1)
    return total


@dataclass
class Item:
    seq: int
    g: int
    n: int
    steps: list           # [(tile key, turn, first, last)] in walk order


@dataclass
class WG:
    xcd: int
    cur: int = -1          # index (in its queue) of the item being processed
    nxt: int = -1          # prefetched index
    step: int = 0
    waiting: object = None


@dataclass
class SimResult:
    makespan: float
    busy: float           # sum of step time over all workgroups
    waited: float         # time workgroups spent blocked on a turn
    deadlock: bool
    items: int


def build_items(lqs, lks, hkv, group, wl, wr, order):
    """Per-XCD item lists.  Pairs (sequence, KV head) in `order` (sequence
    ranks), pair p on queue p % 8, key blocks descending within a pair."""
    nblocks = max(1, max(-(-lk // BN) for lk in lks))
    queues = [[] for _ in range(NXCD)]
    for rank, b in enumerate(order):
        for g in range(hkv):
            pair = rank * hkv + g
            lq, lk = lqs[b], lks[b]
            for n in range(nblocks - 1, -1, -1):
                mb, me = block_tiles(lq, lk, wl, wr, n)
                steps = []
                for i in range((me - mb) * group):
                    m = mb + i // group
                    h = g * group + i % group
                    n_lo, n_hi = contributors_closed(lq, lk, wl, wr, m)
                    steps.append(((b, h, m), n_hi - n, n == n_hi, n == n_lo))
                queues[pair % NXCD].append(Item(b, g, n, steps))
    return queues


def simulate(queues, resident, poll_at=0.9, item_cost=0.5, drain_cost=0.25, empty_cost=0.02, prefetch=False,
             lag=1, max_events=10**7):
    """Discrete-event run of the queues with `resident` workgroups per XCD.

    A step lasts 1.  The dQ partial of step i is read-modify-written at
    fraction `poll_at` of step i + 1 (or in the drain after the last step),
    where the workgroup blocks until the tile's counter equals its turn; the
    tile is released (counter + 1) when that step ends (lag 0) or when the
    next one ends (lag 1: the loads are issued at the poll, the sums stored
    in the next step; the drain then takes two short steps).  Workgroups fetch
    their next item index when they start the item they fetched before
    (`prefetch`), or only when they are free to start it."""
    counters = {}
    waiters = {}          # (tile, turn) -> list of callbacks
    heads = [0] * NXCD    # next index to hand out, per queue
    events = []           # (time, seq, fn)
    seq = [0]
    stats = dict(busy=0.0, waited=0.0, done=0, end=0.0)

    def push(t, fn):
        seq[0] += 1
        heapq.heappush(events, (t, seq[0], fn))

    def fetch(x):
        i = heads[x]
        heads[x] += 1
        return i

    def release(t, tile):
        counters[tile] = counters.get(tile, 0) + 1
        for fn in waiters.pop((tile, counters[tile]), []):
            push(t, fn)

    def start_item(w, t):
        q = queues[w.xcd]
        w.cur = w.nxt if w.nxt >= 0 else fetch(w.xcd)
        w.nxt = -1
        if w.cur >= len(q):
            stats["end"] = max(stats["end"], t)
            return
        if prefetch:
            w.nxt = fetch(w.xcd)
        it = q[w.cur]
        if not it.steps:
            stats["busy"] += empty_cost
            push(t + empty_cost, lambda t2, w=w: finish_item(w, t2))
            return
        stats["busy"] += item_cost
        push(t + item_cost, lambda t2, w=w: run_step(w, t2, 0))

    def finish_item(w, t):
        stats["done"] += 1
        start_item(w, t)

    def run_step(w, t, s):
        it = queues[w.xcd][w.cur]
        nsteps = len(it.steps)
        dur = 1.0 if s < nsteps else drain_cost
        rel = w.waiting      # tile whose sums are stored in this step (lag 1)
        w.waiting = None
        if s == 0 or s > nsteps:   # nothing to poll in this step
            stats["busy"] += dur
            push(t + dur, lambda t2, w=w, s=s, rel=rel: end_step(w, t2, s, rel))
            return
        tile, turn, first, last = it.steps[s - 1]
        t_poll = t + poll_at * dur

        def after_poll(t2, w=w, s=s, tile=tile, last=last, t0=t, dur=dur, rel=rel):
            stats["waited"] += t2 - (t0 + poll_at * dur)
            t_end = t2 + (1 - poll_at) * dur
            stats["busy"] += dur
            mine = None if last else tile
            if lag:
                w.waiting = mine
                push(t_end, lambda t3, w=w, s=s, rel=rel: end_step(w, t3, s, rel))
            else:
                push(t_end, lambda t3, w=w, s=s, rel=rel, mine=mine: (end_step(w, t3, s, rel, mine)))

        if first or counters.get(tile, 0) == turn:
            push(t_poll, after_poll)
        else:
            waiters.setdefault((tile, turn), []).append(after_poll)

    def end_step(w, t, s, rel, rel2=None):
        for r in (rel, rel2):
            if r is not None:
                release(t, r)
        it = queues[w.xcd][w.cur]
        if s + 1 <= len(it.steps) + lag:
            run_step(w, t, s + 1)
        else:
            finish_item(w, t)

    wgs = []
    for x in range(NXCD):
        for _ in range(resident):
            w = WG(x)
            wgs.append(w)
            push(0.0, lambda t, w=w: start_item(w, t))
    n_ev = 0
    while events and n_ev < max_events:
        t, _, fn = heapq.heappop(events)
        fn(t)
        n_ev += 1
    total_items = sum(len(q) for q in queues)
    deadlock = stats["done"] < total_items
    return SimResult(stats["end"], stats["busy"], stats["waited"], deadlock, stats["done"])
