"""Host model of the range kernel's schedule (csrc/maxsim_range.h) and of its combine:
the docs' tiles in doc order cut into equal contiguous ranges per wave. Checked over many
length laws, with empty docs and wave counts from 4 to 3072: every tile is issued exactly
once, each doc is scored exactly once (whole in one wave, or as pieces that the combine
finds), and no two pieces share a slot.

The formulas are the kernel's: W_act = min(W, max(1, T // 2)), wave w's range
[w T // W_act, (w + 1) T // W_act), the wave of tile t = ceil((t + 1) W_act / T) - 1,
head slot w for a piece that opens a range, tail slot W_act + w for one that closes it.
The GPU parity tests exercise the kernels themselves."""

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
