"""Host model of the length-binned schedule's arithmetic, checked over many length
distributions: every doc's tiles are covered exactly once by non-empty chunks, and the
split docs and their chunks fit the workspace slots the library reserves.

This mirrors the formulas the plan and score kernels use (bins by tile count, chunk
size CT = max(2, NQT, ceil(T / (4 W))), ceil(2^b / CT) chunks per doc of bin b); the GPU
parity tests exercise the kernels themselves.
"""

import numpy as np
import pytest

ITEMS_PER_WAVE = 4
NUM_BINS = 28


def bin_of(nt):
    return 0 if nt <= 1 else int(nt - 1).bit_length()


def slots(B, waves):
    """Partial-maxima slots the library reserves (maxsim_common.h, partial_slots_for)."""
    s = 2 * ITEMS_PER_WAVE * waves
    return s + min(B, s)


def schedule(lengths, waves, nqt=1):
    nt = [(int(n) + 15) // 16 for n in lengths]
    T = sum(nt)
    ct = max(2, nqt, -(-T // (waves * ITEMS_PER_WAVE)))
    bins = [[] for _ in range(NUM_BINS)]
    for i, t in enumerate(nt):
        bins[bin_of(t)].append(i)
    items = []  # (claim, desc index, doc, chunk, K, tile range)
    claim = desc = 0
    for b in range(NUM_BINS - 1, -1, -1):
        cap = 1 << b
        K = -(-cap // ct) if cap > ct else 1
        for i in bins[b]:
            for c in range(K):
                items.append((claim, desc, i, c, K, (c * nt[i] // K, (c + 1) * nt[i] // K)))
                claim += 1
            desc += 1
    return nt, items


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("waves", [64, 1024, 8192])
@pytest.mark.parametrize("nqt", [1, 8])
def test_schedule_covers_and_fits(seed, waves, nqt):
    rng = np.random.default_rng(seed)
    kind = seed % 4
    B = int(rng.integers(1, 3000))
    if kind == 0:
        lengths = rng.integers(0, 600, size=B)
    elif kind == 1:
        lengths = np.clip(np.rint(np.exp(rng.normal(np.log(1024), 0.9, size=B))), 0, 60000)
    elif kind == 2:
        lengths = rng.integers(0, 3, size=B) * rng.integers(1, 40000, size=B)
    else:
        lengths = np.full(B, int(rng.integers(1, 5000)))
    nt, items = schedule(lengths, waves, nqt)
    covered = [[] for _ in lengths]
    for claim, desc, i, c, K, (a, b) in items:
        if nt[i] > 0:
            assert b > a, "empty chunk"
        covered[i].append((a, b))
        if K > 1:
            assert desc < 2 * ITEMS_PER_WAVE * waves
            assert desc < len(lengths)
            assert claim < slots(len(lengths), waves)
    for i, rngs in enumerate(covered):
        rngs.sort()
        assert rngs[0][0] == 0 and rngs[-1][1] == nt[i]
        for (a0, b0), (a1, b1) in zip(rngs, rngs[1:]):
            assert b0 == a1


def split_claims(lengths, waves, nqt=1):
    """Number of work items of split docs (slots of per-row maxima the launch writes)."""
    _, items = schedule(lengths, waves, nqt)
    return sum(1 for it in items if it[4] > 1)


@pytest.mark.parametrize("waves", [4, 12, 64, 768, 3072])
@pytest.mark.parametrize("nqt", [1, 2, 8])
def test_slot_bound_adversarial(waves, nqt):
    """Docs of 2^(b-1) + 1 tiles get the most chunks per tile (ceil(2^b / CT) chunks for
    just over half of 2^b tiles); mixed with filler docs that raise or lower T, and with
    B around the 8 W split-doc bound, these come closest to the reserved slot count."""
    rng = np.random.default_rng(waves * 10 + nqt)
    worst = 0.0
    for trial in range(60):
        b = int(rng.integers(1, 14))
        n_big = int(rng.integers(1, 3 * 8 * waves + 2))
        big = np.full(n_big, ((1 << (b - 1)) + 1) * 16 - int(rng.integers(0, 16)))
        n_small = int(rng.integers(0, 2 * waves + 1))
        small = rng.integers(0, 40, size=n_small)
        lengths = np.concatenate([big, small])
        if len(lengths) > 40000:
            lengths = lengths[:40000]
        used = split_claims(lengths, waves, nqt)
        cap = slots(len(lengths), waves)
        assert used <= cap, (b, len(lengths), used, cap)
        worst = max(worst, used / cap)
    assert worst > 0.0
