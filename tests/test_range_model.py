"""Host model of the range kernel's schedule (csrc/maxsim_range.h) and of its combine:
the docs' tiles in doc order cut into equal contiguous ranges per wave. Checked over many
length laws, with empty docs and wave counts from 4 to 3072: every tile is issued exactly
once, each doc is scored exactly once (whole in one wave, or as pieces that the combine
finds), and no two pieces share a slot.

The formulas are the kernel's: W_act = min(W, max(1, T // 2)), wave w's range
[w T // W_act, (w + 1) T // W_act), the wave of tile t = ceil((t + 1) W_act / T) - 1,
head slot w for a piece that opens a range, tail slot W_act + w for one that closes it.
The prologue's search for each range's first doc (per-thread block sums of up to 32
docs, a count of block starts, a scan within the block) is checked against a plain
search over the prefix sums, with its LDS reads inside the region the host sizes. The
GPU parity tests exercise the kernels themselves."""

import numpy as np
import pytest

MIN_TILES = 2


def active(T, W):
    return min(W, max(1, T // MIN_TILES))


def range_start(w, T, wact):
    return (w * T) // wact


def range_wave(t, T, wact):
    return -(-((t + 1) * wact) // T) - 1


def walk(lengths, W):
    """The pieces each wave scores: (wave, doc, first tile, end tile, kind) with kind 0
    whole doc, 1 head slot, 2 tail slot; and the tiles each wave issues."""
    nt = [(int(n) + 15) // 16 for n in lengths]
    S = np.concatenate([[0], np.cumsum(nt)]).astype(np.int64)
    T = int(S[-1])
    wact = active(T, W)
    pieces, issued = [], []
    for w in range(W):
        if w >= wact or T == 0:
            continue
        rb = range_start(w, T, wact)
        re = T if w + 1 == wact else range_start(w + 1, T, wact)
        if re <= rb:
            continue
        doc = int(np.searchsorted(S, rb, side="right") - 1)  # largest i with S_i <= rb
        assert nt[doc] > 0
        pos = rb
        t_begin = rb - int(S[doc])
        while True:
            doc_end = int(S[doc]) + nt[doc]
            t_end = min(doc_end, re) - int(S[doc])
            kind = 1 if t_begin > 0 else (2 if t_end < nt[doc] else 0)
            pieces.append((w, doc, t_begin, t_end, kind))
            issued.extend(int(S[doc]) + t for t in range(t_begin, t_end))
            pos = int(S[doc]) + t_end
            if pos >= re:
                break
            doc += 1
            while nt[doc] == 0:
                doc += 1
            assert int(S[doc]) == pos
            t_begin = 0
    return nt, S, T, wact, pieces, issued


def combine_slots(S, T, wact, doc):
    s, e = int(S[doc]), int(S[doc + 1])
    if e == s:
        return None
    lo, hi = range_wave(s, T, wact), range_wave(e - 1, T, wact)
    if lo == hi:
        return None
    return [wact + lo] + list(range(lo + 1, hi + 1))


def lengths_cases():
    rng = np.random.default_rng(7)
    yield np.array([5])
    yield np.array([0, 0, 0])
    yield np.array([0, 16, 0, 17, 0])
    yield np.full(1024, 1)
    yield np.full(1024, 4096)
    for k in range(40):
        B = int(rng.integers(1, 1025))
        kind = k % 5
        if kind == 0:
            L = rng.integers(0, 300, size=B)
        elif kind == 1:
            L = np.clip(np.rint(np.exp(rng.normal(np.log(1024), 0.6, size=B))), 32, 4096)
        elif kind == 2:
            L = rng.integers(0, 3, size=B) * rng.integers(1, 20000, size=B)
        elif kind == 3:
            L = rng.integers(16, 129, size=B)
        else:
            L = np.where(rng.random(B) < 0.5, 0, rng.integers(1, 40, size=B))
        yield L.astype(np.int64)


@pytest.mark.parametrize("W", [4, 12, 64, 768, 2048, 3072])
def test_every_tile_once_every_doc_once_slots_unique(W):
    for lengths in lengths_cases():
        nt, S, T, wact, pieces, issued = walk(lengths, W)
        assert sorted(issued) == list(range(T))  # each tile issued exactly once
        written = {}
        by_doc = {}
        for w, doc, tb, te, kind in pieces:
            assert te > tb
            by_doc.setdefault(doc, []).append((w, tb, te, kind))
            if kind:
                slot = w if kind == 1 else wact + w
                assert slot not in written, "two pieces in one slot"
                assert slot < 2 * W
                written[slot] = doc
        for doc in range(len(lengths)):
            ps = by_doc.get(doc, [])
            if nt[doc] == 0:
                assert not ps  # empty: no tile; its -inf comes from the prologue
                assert combine_slots(S, T, wact, doc) is None
                continue
            slots = combine_slots(S, T, wact, doc)
            if len(ps) == 1:
                assert ps[0][3] == 0 and ps[0][1:3] == (0, nt[doc])
                assert slots is None
            else:
                assert all(k != 0 for *_, k in ps)
                assert sorted(slots) == sorted(s for s, dd in written.items() if dd == doc)
                cover = sorted((tb, te) for _, tb, te, _ in ps)
                assert cover[0][0] == 0 and cover[-1][1] == nt[doc]
                assert all(b0 == a1 for (_, b0), (a1, _) in zip(cover, cover[1:]))


@pytest.mark.parametrize("T", [1, 2, 3, 7, 100, 4096, 2 ** 20 + 3, 2 ** 31 + 11])
@pytest.mark.parametrize("wact", [1, 3, 64, 3072])
def test_range_wave_inverts_range_start(T, wact):
    if wact > T:
        return
    for w in {0, 1, wact // 2, wact - 1}:
        if w >= wact:
            continue
        rb = range_start(w, T, wact)
        re = T if w + 1 == wact else range_start(w + 1, T, wact)
        for t in {rb, re - 1, (rb + re) // 2}:
            if rb <= t < re:
                assert range_wave(t, T, wact) == w


# ---- the prologue's search for each wave's first doc, for batches of up to 8192 docs

THREADS = 256


def prologue_first_docs(lengths, W):
    """Each active wave's (first doc, its first tile) as the prologue finds them: thread t
    sums the tiles of its block of 4 nch docs chunk by chunk from chunk t mod nch on; the
    blocks' first tiles are their exclusive prefix sums; a wave counts the block starts at
    or below its first tile, then scans its block's docs. Also returns every LDS index the
    prologue reads, for the bounds check."""
    B = len(lengths)
    nch = -(-B // (4 * THREADS))
    dpt = 4 * nch
    nt = np.array([(int(n) + 15) // 16 if n > 0 else 0 for n in lengths] + [0] * (THREADS * dpt - B), np.int64)
    reads = []
    mine = np.zeros(THREADS, np.int64)
    for t in range(THREADS):
        c = t % nch
        for j in range(nch):
            i0 = t * dpt + 4 * c
            reads.extend(range(i0, i0 + 4))
            mine[t] += sum(nt[i] for i in range(i0, i0 + 4) if i < B)
            c = 0 if c + 1 == nch else c + 1
    blk_first = np.concatenate([[0], np.cumsum(mine)[:-1]])
    T = int(mine.sum())
    wact = active(T, W)
    found = {}
    for w in range(min(W, wact)):
        rb = range_start(w, T, wact)
        re = T if w + 1 == wact else range_start(w + 1, T, wact)
        if re <= rb:
            continue
        k = int(np.sum(blk_first <= rb)) - 1
        lane_nt = [nt[k * dpt + l] if k * dpt + l < B else 0 for l in range(dpt)]
        reads.extend(k * dpt + l for l in range(dpt) if k * dpt + l < B)
        incl = np.cumsum(lane_nt)
        first = [int(blk_first[k] + incl[l] - lane_nt[l]) for l in range(dpt)]
        hit = [l for l in range(dpt) if lane_nt[l] > 0 and first[l] <= rb < first[l] + lane_nt[l]]
        assert len(hit) == 1, (w, rb, hit)
        found[w] = (k * dpt + hit[0], first[hit[0]])
    return found, reads, nch


def prologue_cases():
    rng = np.random.default_rng(11)
    yield np.array([7])
    yield np.zeros(5, np.int64)
    yield np.full(8192, 1)
    yield np.full(8192, 512)
    for B in (1023, 1024, 1025, 2048, 3000, 5000, 8191, 8192):
        yield rng.integers(0, 513, size=B)
    for _ in range(6):
        B = int(rng.integers(1, 8193))
        yield np.where(rng.random(B) < 0.7, 0, rng.integers(1, 5000, size=B))


@pytest.mark.parametrize("W", [4, 64, 3072])
def test_prologue_search_finds_each_ranges_first_doc(W):
    for lengths in prologue_cases():
        nt = [(int(n) + 15) // 16 if n > 0 else 0 for n in lengths]
        S = np.concatenate([[0], np.cumsum(nt)]).astype(np.int64)
        T = int(S[-1])
        found, reads, nch = prologue_first_docs(lengths, W)
        if T == 0:
            assert not found
            continue
        wact = active(T, W)
        for w, (doc, first_tile) in found.items():
            rb = range_start(w, T, wact)
            want = int(np.searchsorted(S, rb, side="right") - 1)  # largest i with S_i <= rb
            assert doc == want and first_tile == int(S[want]) and nt[doc] > 0
        # every length the prologue reads lies in the LDS region the host sizes for it
        assert max(reads) < 4 * THREADS * nch
