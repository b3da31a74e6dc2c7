"""Docs stored as FP8 E4M3 bytes with one scale (maxsim_rerank_fp8), on the GPU, against
the oracle's FP8 path: |gpu - oracle| <= 1e-3 (1 + |oracle|) per doc, -inf where the
oracle has it. Exact inputs (one-hot queries over every finite E4M3 byte) must match bit
for bit, which pins the hardware E4M3 conversion (format, subnormals, sign, byte order)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

if torch.cuda.is_available():
    import late_interaction_reranking_amd as lir
    from devio import DEV, assert_parity, gpu_scores, upload8


def _say(msg):
    print(msg, flush=True)


def fp8_scores(w, staged=False):
    Q, X8, offs, lens = upload8(w)
    if staged:
        ws = torch.empty(lir.maxsim_workspace_size(w.Lq, w.d, w.B), dtype=torch.uint8, device=DEV)
        lir.maxsim_plan(offs, lens, w.Lq, w.d, ws)
        s = lir.maxsim_score_fp8(Q, X8, offs, lens, w.doc_scale, ws)
        lir.maxsim_finish_fp8(Q, w.B, w.doc_scale, ws, s)
    else:
        s = lir.maxsim_rerank_fp8(Q, X8, offs, lens, w.doc_scale)
    torch.cuda.synchronize()
    return s.cpu().numpy().astype(np.float64)


FINITE = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("d", [16, 128, 96])
def test_fp8_one_hot_every_byte_exact(fmt, d):
    _say(f"[fp8] one-hot all bytes {fmt} d={d}")
    rng = np.random.default_rng([d, len(fmt)])
    Lq = 6
    lengths = rng.integers(0, 40, size=80)
    lengths[:3] = [0, 1, 17]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=d, order="shuffled", gap=(0, 3), gap_fill="nan")
    workloads.to_fp8(w, doc_scale=1.0, stride8=d + 16)
    for o_, n in zip(w.offsets, w.lengths):
        w.X8[o_:o_ + n, :d] = rng.choice(FINITE, size=(n, d))
    # every finite byte in some doc row
    o0 = int(w.offsets[np.argmax(w.lengths)])
    flat = w.X8[o0:o0 + int(w.lengths.max()), :d].reshape(-1)
    flat[: FINITE.size] = FINITE
    w.X8[o0:o0 + int(w.lengths.max()), :d] = flat.reshape(-1, d)
    a = rng.integers(0, d, size=Lq)
    a[0] = 0
    w.Q = np.zeros((Lq, d), np.uint16)
    w.Q[np.arange(Lq), a] = 0x3C00 if fmt == "f16" else 0x3F80
    assert np.array_equal(fp8_scores(w), oracle.maxsim_workload(w))


@pytest.mark.parametrize("name", ["tiny", "colbert", "long_doc", "scattered"])
def test_fp8_named_workloads(name):
    _say(f"[fp8] workload {name}")
    w = workloads.to_fp8(workloads.make(name), doc_scale=1 / 300)
    got = fp8_scores(w)
    ref = oracle.maxsim_workload(w)
    assert_parity(got, ref, name)


SHAPES = [(32, 16, 16), (7, 32, 48), (37, 48, 64), (32, 128, 128), (128, 128, 144), (200, 96, 96),
          (64, 256, 256), (129, 256, 272), (17, 160, 176)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,d,stride8", SHAPES)
def test_fp8_shapes_ragged(fmt, Lq, d, stride8):
    _say(f"[fp8] shape Lq={Lq} d={d} stride={stride8} {fmt}")
    rng = np.random.default_rng([Lq, d, stride8])
    lengths = rng.integers(0, 90, size=60)
    lengths[:8] = [0, 1, 15, 16, 17, 31, 32, 33]
    w = workloads.custom(Lq, d, lengths, dtype=fmt, seed=Lq + d, order="shuffled", gap=(0, 5), gap_fill="nan")
    workloads.to_fp8(w, doc_scale=0.0123, stride8=stride8)
    assert_parity(fp8_scores(w), oracle.maxsim_workload(w), f"Lq={Lq} d={d}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_long_docs_and_staged(fmt):
    _say(f"[fp8] long docs {fmt}")
    lengths = np.array([4096, 4095, 1, 2049, 0, 3000, 17, 5000, 16, 8191])
    w = workloads.custom(64, 128, lengths, dtype=fmt, seed=3, order="shuffled", gap=(1, 3), gap_fill="nan")
    workloads.to_fp8(w, doc_scale=0.004)
    a = fp8_scores(w)
    assert_parity(a, oracle.maxsim_workload(w), "long docs")
    assert np.array_equal(a, fp8_scores(w, staged=True))


def test_fp8_equals_fp16_path_on_exact_values():
    """Doc values scale * e4m3 with a power-of-two scale are exact in fp16: the FP8 path
    and the fp16 path see the same numbers and must agree bit for bit."""
    _say("[fp8] equals fp16 path")
    w = workloads.custom(32, 128, np.random.default_rng(4).integers(1, 300, size=500), seed=4,
                         order="shuffled", gap=(0, 2))
    workloads.to_fp8(w, doc_scale=2.0 ** -8)
    dec = torch.from_numpy(w.X8[:, : w.d]).view(torch.float8_e4m3fn).to(torch.float32).numpy() * w.doc_scale
    dec[np.isnan(dec)] = 0.0
    w16 = workloads.Workload(**{**w.__dict__, "X": np.ascontiguousarray(dec.astype(np.float16)).view(np.uint16),
                                "stride": w.d, "X8": None, "doc_scale": 1.0})
    assert np.array_equal(fp8_scores(w), gpu_scores(w16))


def test_fp8_scale_is_linear():
    _say("[fp8] scale")
    w = workloads.to_fp8(workloads.colbert(), doc_scale=2.0 ** -8)
    a = fp8_scores(w)
    w.doc_scale = 2.0 ** -5
    assert np.array_equal(fp8_scores(w), a * 8.0)


def test_fp8_errors_raise():
    _say("[fp8] errors")
    w = workloads.to_fp8(workloads.tiny(), doc_scale=0.01)
    Q, X8, offs, lens = upload8(w)
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_rerank_fp8(Q, X8, offs, lens, 0.0)
    with pytest.raises(TypeError):
        lir.maxsim_rerank_fp8(Q, X8.to(torch.float16), offs, lens, 1.0)
    with pytest.raises(TypeError):
        lir.maxsim_rerank_fp8(Q.float(), X8, offs, lens, 1.0)
    Q48 = torch.zeros((4, 40), dtype=torch.float16, device=DEV)
    X40 = torch.zeros((100, 48), dtype=torch.uint8, device=DEV)[:, :40]
    with pytest.raises(lir.MaxSimError):
        lir.maxsim_rerank_fp8(Q48, X40, offs, lens, 1.0)  # d % 16


@pytest.mark.slow
def test_fp8_large_sampled():
    _say("[fp8] large_fp8 (generating)")
    w = workloads.make("large_fp8")
    got = fp8_scores(w)
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([w.planted, rng.choice(w.B, 3000, replace=False), [0, w.B - 1]]))
    assert_parity(got[sample], oracle.maxsim_workload(w, docs=sample), "large_fp8 (sample)")


# ------------------------------------------------------------------ batch forms


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_pairs_batch(fmt):
    _say(f"[fp8] pairs {fmt}")
    rng = np.random.default_rng(31)
    q_lengths = rng.integers(0, 65, size=9)
    q_lengths[:2] = [0, 64]
    per = rng.integers(0, 30, size=9)
    lengths = rng.integers(0, 300, size=int(per.sum()))
    lengths[rng.choice(lengths.size, 3, replace=False)] = [3000, 4500, 6000]
    w = workloads.custom_pairs(q_lengths, 96, per, lengths, dtype=fmt, seed=31, interleave=True,
                               order="shuffled", gap=(0, 4), gap_fill="nan")
    workloads.to_fp8(w, doc_scale=0.02)
    Q, X8, offs, lens = upload8(w)
    got = lir.maxsim_rerank_pairs_fp8(Q, _i32(w.q_offsets), _i32(w.q_lengths), w.Lq, X8, offs, lens,
                                      _i32(w.doc_query), w.doc_scale).cpu().numpy().astype(np.float64)
    ref = oracle.maxsim_workload(w)
    assert_parity(got, ref, f"fp8 pairs {fmt}")
    for j in range(w.nq):  # each doc equals its query scored alone
        sel = np.nonzero(w.doc_query == j)[0]
        if not sel.size:
            continue
        lo, n = int(w.q_offsets[j]), int(w.q_lengths[j])
        Qj = Q[lo:lo + n].contiguous()
        alone = lir.maxsim_rerank_fp8(Qj, X8, offs[sel].contiguous(), lens[sel].contiguous(), w.doc_scale)
        assert np.array_equal(got[sel], alone.cpu().numpy().astype(np.float64)), j


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fp8_shared_docs(fmt):
    _say(f"[fp8] shared docs {fmt}")
    rng = np.random.default_rng(32)
    q_lengths = [32, 0, 17, 32, 100, 5, 32]
    lengths = rng.integers(0, 300, size=150)
    lengths[:3] = [0, 5000, 1]
    w = workloads.custom_multi(q_lengths, 128, lengths, dtype=fmt, seed=32, order="shuffled", gap=(0, 3),
                               gap_fill="nan")
    workloads.to_fp8(w, doc_scale=1 / 128)
    Q, X8, offs, lens = upload8(w)
    got = lir.maxsim_rerank_multi_fp8(Q, w.q_lengths, X8, offs, lens, w.doc_scale).cpu().numpy().astype(np.float64)
    ref = oracle.maxsim_workload(w)
    lo = 0
    for j, n in enumerate(q_lengths):
        assert_parity(got[j], ref[j], f"fp8 shared query {j}")
        alone = lir.maxsim_rerank_fp8(Q[lo:lo + n].contiguous(), X8, offs, lens, w.doc_scale)
        assert np.array_equal(got[j], alone.cpu().numpy().astype(np.float64)), j
        lo += n
