"""CPU checks of the fused backward's ordered dQ reduction (host-side model in
dq_order_model.py, written independently of the kernel source).

1. The closed form that gives each query tile its contributing key blocks
   (used by the kernel to find a workgroup's turn) matches a brute-force walk
   of every block's query range, over causal, non-causal, windowed and
   cross-attention shapes (Lq != Lk, bottom-right alignment).
2. The per-XCD queues and turn waits cannot deadlock: the event simulation
   finishes every item for 1..32 resident workgroups per XCD on the length
   draws of the jagged, full-length and short-KV workloads, under each mask.
3. Every allowed (query, key) pair is covered by exactly one contributor of
   its query tile (no pair counted twice or missed by the tile ranges).
"""
import numpy as np
import pytest

import dq_order_model as M
import gdpa_inputs as gi

MASKS = [(-1, -1), (-1, 0), (511, 0), (0, 0), (3, 4), (-1, 40), (100, -1), (0, -1), (130, 70)]


def test_closed_form_contributors_match_brute_force():
    lens = list(range(0, 300, 7)) + [64, 127, 128, 129, 1024, 2047, 2048]
    for lq in lens:
        for lk in lens:
            for wl, wr in MASKS:
                brute = M.contributors_brute(lq, lk, wl, wr)
                for m, blocks in brute.items():
                    lo, hi = M.contributors_closed(lq, lk, wl, wr, m)
                    assert blocks == (list(range(lo, hi + 1)) if lo <= hi else []), (lq, lk, wl, wr, m)


def test_tiles_cover_every_allowed_pair_once():
    # each allowed (query i, key j) pair lies in the walk of exactly the key
    # block that holds j, and that block lists i's tile among its tiles
    rng = np.random.default_rng(7)
    for _ in range(60):
        lq, lk = int(rng.integers(0, 400)), int(rng.integers(0, 400))
        wl, wr = MASKS[int(rng.integers(len(MASKS)))]
        off = lk - lq
        for i in range(lq):
            lo = 0 if wl < 0 else max(0, i + off - wl)
            hi = lk - 1 if wr < 0 else min(lk - 1, i + off + wr)
            for j in range(lo, hi + 1):
                b, e = M.block_tiles(lq, lk, wl, wr, j // M.BN)
                assert b <= i // M.BQ < e, (lq, lk, wl, wr, i, j)


def _draw(name, seed=None):
    wl = gi.WORKLOADS[name]
    lq, lk = gi.draw_seqlens(wl, seed)
    lq = [int(x) for x in lq]
    lk = [int(x) for x in lk]
    order = list(np.argsort(-(np.array(lq) + np.array(lk)), kind="stable")) if wl.varlen else list(range(len(lq)))
    return wl, lq, lk, order


@pytest.mark.parametrize("name", ["jagged_self", "full_self", "short_kv_cross", "window_gqa_fp8"])
@pytest.mark.parametrize("mask", [(-1, -1), (-1, 0), (511, 0), (0, 0)])
def test_queues_and_turn_waits_do_not_deadlock(name, mask):
    wl, lq, lk, order = _draw(name)
    # a prefix of the batch keeps the run short (8 full-length sequences, 48
    # of the others); the per-pair structure is the workload's
    keep = 8 if name == "full_self" else 48
    order = [b for b in order if b < keep]
    queues = M.build_items(lq, lk, wl.heads_kv, wl.heads_q // wl.heads_kv, mask[0], mask[1], order)
    for resident in (1, 3, 8, 32):
        r = M.simulate(queues, resident)
        assert not r.deadlock, (name, mask, resident, r.items)
        assert r.items == sum(len(q) for q in queues)


def test_every_resident_count_on_a_small_batch():
    # all of 1..32 resident workgroups per XCD, ragged lengths, GQA 2:1
    rng = np.random.default_rng(11)
    lq = [int(x) for x in rng.integers(0, 700, size=24)]
    lk = [int(x) for x in rng.integers(0, 700, size=24)]
    order = list(np.argsort(-(np.array(lq) + np.array(lk)), kind="stable"))
    for mask in [(-1, -1), (-1, 0), (200, 0)]:
        queues = M.build_items(lq, lk, 2, 2, mask[0], mask[1], order)
        for resident in range(1, 33):
            r = M.simulate(queues, resident)
            assert not r.deadlock, (mask, resident)


def test_length_draw_matches_make_batch():
    wl = gi.small_variant(gi.WORKLOADS["short_kv_cross"], 6, (3, 40), (5, 9))
    bt = gi.make_batch(wl)
    lq, lk = gi.draw_seqlens(wl)
    assert list(lq) == list(bt.seqlens_q) and list(lk) == list(bt.seqlens_k)
