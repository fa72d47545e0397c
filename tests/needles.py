"""Positions for planted dominant keys in long-context decode tests.

With N(0, 1) keys over tens of thousands of tokens the softmax is nearly flat, outputs are about 1/sqrt(L) in
size and sit under the bf16 tolerance's absolute term: a decode that dropped or repeated whole tiles would
still pass. ``workloads.plant_dominant_keys`` fixes that: each query head gets two planted keys of equal,
dominant score, so its output is the mean of those two tokens' values (the other tokens weigh below e^-36).
Dropping either planted token moves the output to the other's value; counting one twice moves it to
(2 v_a + v_b) / 3. Either way it moves by about |v_a - v_b| / 6 or more, far outside the tolerance
(``tests/test_needles.py`` shows this with the oracle alone).

The positions sweep what a kernel could get wrong: the first and last token of a sequence, of 32-token tiles,
of blocks and of the parts the decode plan cuts a sequence into. Part bounds come from ``plan_parts``, a host
restatement of the plan's documented rule; if it ever drifted from the device's cut, the positions would still
be valid tile boundaries, only less targeted.
"""
from __future__ import annotations

import numpy as np

TILE = 32


def _cdiv(a, b):
    return -(-int(a) // int(b))


def plan_parts(lens, num_kv_heads, block_size, workers, min_strata=1, min_tiles=4):
    """Parts (seq, first token, tokens) of the decode plan's cut for ``workers`` resident waves.

    The rule: t_i = ceil(L_i / 32) tiles; g = clamp(ceil(Hkv sum t_i / cap), min_tiles, max_tiles) with
    cap = min_strata * workers and max_tiles the tiles whose block-table slice fits 64 lanes (64 blocks, or 63
    when blocks are longer than a tile); n_i = max(1, round(t_i / g), ceil(t_i / max_tiles)), parts of
    32 ceil(t_i / n_i) tokens, the last taking the rest. When every sequence fits one unit per wave but the cut
    makes more than cap units, g grows to max(g + 1, ceil(g U / cap)) and the cut is redone."""
    lens = [max(0, int(x)) for x in lens]
    hkv, cap = int(num_kv_heads), int(workers) * int(min_strata)
    max_tiles = (64 if block_size <= TILE else 63) * int(block_size) // TILE
    tiles = [_cdiv(n, TILE) for n in lens]
    target = min(max(_cdiv(hkv * sum(tiles), cap), min_tiles), max_tiles)
    fits = hkv * sum(_cdiv(t, max_tiles) for t in tiles) <= cap
    while True:
        cut = []
        for t in tiles:
            if t == 0:
                cut.append((0, 0))
                continue
            n = max(max(1, (t + target // 2) // target), _cdiv(t, max_tiles))
            lt = _cdiv(t, n)
            cut.append((_cdiv(t, lt), lt * TILE))
        total = sum(n for n, _ in cut)
        if hkv * total <= cap or target >= max_tiles or len(lens) * hkv > cap or not fits:
            break
        grown = _cdiv(target * hkv * total, cap)
        target = min(max(grown, target + 1), max_tiles)
    parts = []
    for i, ((n, plen), L) in enumerate(zip(cut, lens)):
        for p in range(n):
            start = p * plen
            parts.append((i, start, min(plen, L - start)))
    return parts


def boundary_positions(L, block_size, parts_of_seq):
    """Candidate positions of one sequence by kind: its ends, tile bounds, block bounds, part bounds."""
    L = int(L)
    if L == 0:
        return {}
    ends = [0, L - 1]
    tile = sorted({x for k in range(0, L, TILE) for x in (k, k + TILE - 1) if x < L})
    block = sorted({x for k in range(0, L, block_size) for x in (k, k + block_size - 1) if x < L})
    part = sorted({x for s, n in parts_of_seq for x in (s, s + n - 1) if 0 <= x < L})
    return {"ends": ends, "tile": tile, "block": block, "part": part}


def needle_positions(case, rng, workers, per_head=2):
    """positions[i][h] for ``workloads.plant_dominant_keys``: ``per_head`` distinct positions per query head,
    distinct across the heads of a kv head, drawn in turn from the part, block, tile and end bounds of each
    sequence; a head's positions are spread over the sequence (the sorted picks are paired first half with
    second half, so they fall in different tiles whenever the sequence allows). Sequences shorter than
    per_head * G tokens plant fewer heads."""
    g = case.num_heads // case.num_kv_heads
    parts = plan_parts(case.context_lens, case.num_kv_heads, case.block_size, workers)
    by_seq = {}
    for i, s, n in parts:
        by_seq.setdefault(i, []).append((s, n))
    out = []
    for i in range(case.num_seqs):
        L = int(case.context_lens[i])
        cands = boundary_positions(L, case.block_size, by_seq.get(i, []))
        heads = [[] for _ in range(case.num_heads)]
        k_per = per_head if L >= per_head * g else (1 if L >= g else 0)
        if k_per:
            order = ["part", "block", "tile", "ends"]
            for kvh in range(case.num_kv_heads):
                need, chosen, seen, k = k_per * g, [], set(), 0
                while len(chosen) < need and k < 200 * need:
                    pool = cands[order[k % len(order)]]
                    k += 1
                    if pool:
                        t = int(pool[rng.integers(len(pool))])
                        if t not in seen:
                            seen.add(t)
                            chosen.append(t)
                while len(chosen) < need:                       # short sequences: any free position
                    t = int(rng.integers(L))
                    if t not in seen:
                        seen.add(t)
                        chosen.append(t)
                chosen.sort()
                for j in range(g):
                    heads[kvh * g + j] = [chosen[j + r * g] for r in range(k_per)]
        out.append(heads)
    return out


def rel_norm_err(got, ref):
    """||got - ref|| / ||ref|| over all elements."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
