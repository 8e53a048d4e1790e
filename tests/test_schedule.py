"""Host-side checks of the persistent tile order (fa_schedule; CPU only).

The order is the FlashAttention-4 paper's longest-processing-time-first
schedule (section 3.3): every tile is processed exactly once, the cost of
the tiles a worker meets never increases from one round to the next for
dense causal masking (m-blocks in reverse; varlen causal batches keep the
order of their rounds and pair each round greedily), and the makespan is
close to the ideal total/workers.
"""
import math

import numpy as np
import pytest

import exact_attention_forward_04_amd as fa
from attn_inputs import WORKLOADS, make, varlen_lengths, cu_seqlens_of

BN = 64


def tile_cost(code, H, S, bm, causal, lens):
    nmb = math.ceil(S / bm)
    mb = code % nmb
    b = code // (nmb * H)
    L = lens[b]
    kv = min(L, (mb + 1) * bm) if causal else L
    return math.ceil(kv / BN)


def all_tiles(B, H, S, bm, lens):
    nmb = math.ceil(S / bm)
    out = set()
    for b in range(B):
        for h in range(H):
            for mb in range(math.ceil(lens[b] / bm)):
                out.add((b * H + h) * nmb + mb)
    return out


CASES = [
    # (B, H, S, D, causal, lens or None, workers)
    (2, 16, 2048, 128, True, None, 256),
    (2, 16, 2048, 128, False, None, 256),
    (1, 16, 32768, 128, True, None, 256),
    (2, 16, 8192, 128, True, None, 256),
    (2, 16, 8192, 256, False, None, 256),
    (2, 16, 8192, 192, True, None, 256),     # (192, 128) head dimensions
    (1, 8, 512, 64, True, None, 256),
    (1, 2, 128, 64, False, None, 256),
    (3, 5, 1000, 128, True, None, 256),      # H not a multiple of 8
    (3, 5, 1000, 128, True, None, 13),       # workers not a multiple of 8
    (16, 32, 8192, 128, True, "C4", 256),
    (5, 8, 3000, 128, True, [1, 0, 3000, 257, 999], 256),
    (5, 8, 3000, 128, False, [1, 0, 3000, 257, 999], 256),
]


@pytest.mark.parametrize("case", CASES)
def test_every_tile_exactly_once(case):
    B, H, S, D, causal, lens, workers = case
    if lens == "C4":
        lens = list(varlen_lengths(16, 512, 8192, WORKLOADS["varlen_16x512to8192_h32d128_causal"].seed))
        S = max(lens)
    cu = None if lens is None else cu_seqlens_of(lens)
    L = [S] * B if lens is None else list(lens)
    tiles, bm = fa.schedule(B, H, S, D, causal, workers, cu_seqlens=cu)
    seen = tiles[tiles >= 0].tolist()
    assert len(seen) == len(set(seen)), "a tile is processed twice"
    assert set(seen) == all_tiles(B, H, S, bm, L), "a tile is missing or foreign"
    # idle slots only at the end of a worker's list
    for row in tiles:
        idle = np.flatnonzero(row < 0)
        if idle.size:
            assert np.all(row[idle[0]:] < 0)
    # LPT (causal): within each worker the costs never increase.  Varlen
    # causal batches are ordered by chunks of `sub` levels (the m-blocks of
    # one sequence run together for K/V reuse in L2): there the chunk of a
    # worker's tiles never goes back, and inside a chunk costs differ by at
    # most sub-1 m-blocks.
    if causal and lens is not None:
        nmb = math.ceil(S / bm)
        groups = 8 if H % 8 == 0 and workers % 8 == 0 else 1
        sub = min(max((workers // groups) // (H // groups), 1), 8)
        for row in tiles:
            ch = [(nmb - 1 - t % nmb) // sub for t in row if t >= 0]
            assert all(ch[i] <= ch[i + 1] for i in range(len(ch) - 1)), ch
    elif causal:
        for row in tiles:
            c = [tile_cost(t, H, S, bm, causal, L) for t in row if t >= 0]
            assert all(c[i] >= c[i + 1] for i in range(len(c) - 1)), c


@pytest.mark.parametrize("case", [c for c in CASES if c[4]])
def test_makespan_near_ideal(case):
    B, H, S, D, causal, lens, workers = case
    if lens == "C4":
        lens = list(varlen_lengths(16, 512, 8192, WORKLOADS["varlen_16x512to8192_h32d128_causal"].seed))
        S = max(lens)
    cu = None if lens is None else cu_seqlens_of(lens)
    L = [S] * B if lens is None else list(lens)
    tiles, bm = fa.schedule(B, H, S, D, causal, workers, cu_seqlens=cu)
    per_worker = [sum(tile_cost(t, H, S, bm, causal, L) + 2 for t in row if t >= 0) for row in tiles]
    total = sum(per_worker)
    ideal = max(total / workers, max(tile_cost(t, H, S, bm, causal, L) + 2
                                      for t in tiles.ravel() if t >= 0))
    ratio = max(per_worker) / ideal
    # small problems cannot be balanced better than one round of tiles
    rounds = tiles.shape[1]
    assert ratio <= (1.10 if rounds >= 4 else 1.6), (ratio, rounds)


def test_xcd_grouping_keeps_heads_on_one_xcd():
    # H % 8 == 0: worker w (XCD w % 8) only sees heads h with h % 8 == w % 8
    B, H, S = 2, 16, 8192
    tiles, bm = fa.schedule(B, H, S, 128, True, 256)
    nmb = math.ceil(S / bm)
    for w, row in enumerate(tiles):
        for t in row[row >= 0]:
            h = (t // nmb) % H
            assert h % 8 == w % 8


GQA_CASES = [
    # (B, H, H_kv, S, D, causal, lens or None, workers)
    (2, 32, 8, 8192, 128, True, None, 256),      # K/V heads a multiple of 8: grouped by K/V head
    (2, 32, 16, 4096, 128, False, None, 256),
    (1, 32, 4, 8192, 128, True, None, 256),      # fewer K/V heads than XCDs
    (1, 16, 1, 4096, 64, True, None, 256),       # multi-query
    (5, 24, 8, 3000, 128, True, [1, 0, 3000, 257, 999], 256),
    (3, 12, 3, 1000, 128, True, None, 13),
]


@pytest.mark.parametrize("case", GQA_CASES)
def test_gqa_every_tile_exactly_once_and_lpt(case):
    B, H, H_kv, S, D, causal, lens, workers = case
    cu = None if lens is None else cu_seqlens_of(lens)
    L = [S] * B if lens is None else list(lens)
    tiles, bm = fa.schedule(B, H, S, D, causal, workers, cu_seqlens=cu, H_kv=H_kv)
    seen = tiles[tiles >= 0].tolist()
    assert len(seen) == len(set(seen)), "a tile is processed twice"
    assert set(seen) == all_tiles(B, H, S, bm, L), "a tile is missing or foreign"
    if causal and lens is not None:
        # varlen causal: rounds in chunk order, paired greedily inside a round
        nmb = math.ceil(S / bm)
        groups = 8 if H % 8 == 0 and workers % 8 == 0 else 1
        sub = min(max((workers // groups) // (H // groups), 1), 8)
        for row in tiles:
            ch = [(nmb - 1 - t % nmb) // sub for t in row if t >= 0]
            assert all(ch[i] <= ch[i + 1] for i in range(len(ch) - 1)), ch
    elif causal:
        for row in tiles:
            c = [tile_cost(t, H, S, bm, causal, L) for t in row if t >= 0]
            assert all(c[i] >= c[i + 1] for i in range(len(c) - 1)), c


def test_varlen_greedy_rounds_balance():
    """Varlen causal batches pair each round's positions greedily (costliest
    tile to the least-loaded worker of the XCD group): on the 16-sequence
    batch the busiest worker carries at most 1% more than the mean, where
    the fixed snake pairing of the same rounds gave 6.4% more."""
    lens = list(varlen_lengths(16, 512, 8192, WORKLOADS["varlen_16x512to8192_h32d128_causal"].seed))
    B, H, S = 16, 32, max(lens)
    tiles, bm = fa.schedule(B, H, S, 128, True, 256, cu_seqlens=cu_seqlens_of(lens))
    per_worker = [sum(tile_cost(t, H, S, bm, True, lens) + 2.5 for t in row if t >= 0)
                  for row in tiles]
    assert max(per_worker) / np.mean(per_worker) <= 1.01


def test_gqa_query_heads_of_a_kv_head_share_an_xcd():
    # H_kv % 8 == 0: worker w (XCD w % 8) only sees query heads whose K/V head
    # is congruent to w mod 8, and consecutive positions walk the query heads
    # of one K/V head before moving to the next
    B, H, H_kv, S = 2, 32, 8, 8192
    G = H // H_kv
    tiles, bm = fa.schedule(B, H, S, 128, True, 256, H_kv=H_kv)
    nmb = math.ceil(S / bm)
    for w, row in enumerate(tiles):
        for t in row[row >= 0]:
            h = (t // nmb) % H
            assert (h // G) % 8 == w % 8
    # round 0 of the workers of XCD 0 (workers 0, 8, 16, ...): G consecutive
    # workers hold the G query heads of one K/V head
    first = [tiles[w, 0] for w in range(0, 256, 8)]
    heads = [(t // nmb) % H for t in first]
    for i in range(0, len(heads) - G + 1, G):
        assert len({h // G for h in heads[i:i + G]}) == 1, heads


def test_gqa_schedule_rejects_bad_kv_heads():
    with pytest.raises(fa.FaError):
        fa.schedule(1, 12, 1024, 128, True, 256, H_kv=5)


def test_schedule_rejects_small_round_budget():
    with pytest.raises(fa.FaError):
        fa.schedule(1, 16, 32768, 128, True, 256, max_rounds=2)


def test_qk_lengths_order_ranks_by_key_length():
    """Causal batches with key lengths of their own (bottom-right aligned):
    a query tile sees nearly all of its sequence's keys, so the order ranks
    sequences by key length; every tile still runs exactly once and the
    makespan under the key-length cost stays near the ideal."""
    from attn_inputs import qk_lengths
    w = WORKLOADS["mixed_16x_q1to2048_k512to8192_h16d128_causal"]
    lq, lk = qk_lengths(w)
    B, H, S = len(lq), w.H, max(lq)
    tiles, bm = fa.schedule(B, H, S, w.D, True, 256, cu_seqlens=cu_seqlens_of(lq),
                            cu_seqlens_k=cu_seqlens_of(lk))
    seen = tiles[tiles >= 0].tolist()
    assert len(seen) == len(set(seen))
    assert set(seen) == all_tiles(B, H, S, bm, list(lq))
    nmb = math.ceil(S / bm)

    def cost(t):
        b, mb = t // (nmb * H), t % nmb
        last_key = lk[b] - lq[b] + min((mb + 1) * bm, lq[b])   # bottom-right causal
        return math.ceil(min(lk[b], max(0, last_key)) / BN) + 2

    per_worker = [sum(cost(t) for t in row if t >= 0) for row in tiles]
    ideal = max(sum(per_worker) / len(per_worker), max(cost(t) for t in seen))
    assert max(per_worker) / ideal <= 1.15, max(per_worker) / ideal


def test_schedule_general_rejects_one_sided_key_offsets():
    with pytest.raises(fa.FaError):
        import ctypes
        cu = np.array([0, 10], dtype=np.int32)
        tiles = np.zeros((8, 16), dtype=np.int32)
        r, b = ctypes.c_int(0), ctypes.c_int(0)
        fa._check("fa_schedule_general", fa.load().fa_schedule_general(
            1, 8, 8, 10, 128, 1, cu.ctypes.data, None, 8, tiles.ctypes.data, 16,
            ctypes.byref(r), ctypes.byref(b)))


# ---- dense causal split levels

SPLIT_CASES = [
    # (B, H, S, D, nsplit)
    (2, 16, 2048, 128, 8),
    (2, 16, 2048, 128, 3),
    (1, 16, 4096, 128, 16),
    (2, 3, 700, 128, 2),
    (1, 8, 3000, 192, 12),
    (1, 2, 900, 64, 2),
    (2, 16, 1500, 192, 3),
]


def split_part_blocks(mb, part, S, BM):
    """Key blocks (of 64) a part reads: the whole causal range of m-block mb,
    its first floor(n/2) blocks, or the rest."""
    n = -(-min((mb + 1) * BM, S) // 64)
    return n if part == 0 else (n // 2 if part == 1 else n - n // 2)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B%dH%dS%dD%d_n%d" % c)
def test_split_schedule_covers_every_part_once(case):
    """Every unsplit tile runs once whole; each of the nsplit costliest
    m-blocks of every (sequence, head) runs once as part 1 and once as
    part 2, and never whole."""
    B, H, S, D, nsplit = case
    items, BM = fa.schedule_split(B, H, S, D, nsplit, 256)
    nmb = -(-S // BM)
    got = sorted(items[items >= 0].tolist())
    want = []
    for b in range(B):
        for h in range(H):
            for mb in range(nmb):
                base = ((b * H + h) * nmb + mb) * 3
                want += [base + 1, base + 2] if mb >= nmb - nsplit else [base]
    assert got == sorted(want)


def test_split_schedule_shortens_the_busiest_worker():
    """On a one-sequence 2k causal batch (B=1, H=16: half the workers idle
    unsplit) the library splits levels, and its order's busiest worker
    carries less than the unsplit order's (cost units: two per key block,
    five per tile, 18 more per part for the exchange of partial rows)."""
    B, H, S, D = 1, 16, 2048, 128
    n = fa.split_plan(B, H, S, D, 256)
    assert n > 0

    def busiest(nsplit):
        items, BM = fa.schedule_split(B, H, S, D, nsplit, 256)
        nmb = -(-S // BM)
        worst = 0
        for row in items:
            load = 0
            for code in row[row >= 0].tolist():
                part, mb = code % 3, (code // 3) % nmb
                load += 2 * split_part_blocks(mb, part, S, BM) + 5 + (18 if part else 0)
            worst = max(worst, load)
        return worst

    assert busiest(n) <= 0.85 * busiest(0)


def test_split_plan_leaves_large_batches_whole():
    """Batches that fill the workers (the 2k, 8k and 32k causal workloads)
    are not split by default; a request is clamped to what the schedule
    holds (every m-block, at most 64 levels in all)."""
    for B, H, S in ((1, 16, 32768), (2, 16, 8192), (64, 64, 2048), (2, 16, 2048)):
        assert fa.split_plan(B, H, S, 128, 256) == 0
    assert fa.split_plan(2, 16, 2048, 128, 256, requested=100) == 8
    assert fa.split_plan(2, 16, 2048, 128, 256, requested=0) == 0
    assert fa.split_plan(1, 16, 16384, 128, 256, requested=5) == 0  # 64 m-blocks: no room
    with pytest.raises(RuntimeError):
        fa.schedule_split(2, 16, 2048, 128, 9, 256)  # more than the schedule holds
    # D = 256: its pipelined body takes the whole LDS, so it never splits
    assert fa.split_plan(1, 8, 3000, 256, 256) == 0
    assert fa.split_plan(1, 8, 3000, 256, 256, requested=4) == 0
    with pytest.raises(RuntimeError):
        fa.schedule_split(1, 8, 3000, 256, 2, 256)
