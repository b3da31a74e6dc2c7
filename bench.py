"""Benchmark: MaxSim rerank throughput on one MI355X.

One step = the whole hot path over one batch: the length-binned schedule (two plan
kernels), the score kernel and the combine kernel (scores of split docs), for one query
against every doc of the workload, inputs already resident in HBM. HIP events on the
launching stream bracket the score kernel alone for the roofline figures. Prints ONE
JSON line.

Default workload: "large" -- Lq 32, d 128, 80,000 fp16 docs of U[64,448] rows packed
back to back (~20.5 M doc rows, 5.24 GB; row offset * d passes 2^31), 1 % of docs
holding a planted near-duplicate of a query row.

--workload pairs times the multi-query form instead: 64 queries (lengths U[16,32]) with
1000 ColBERT-shaped docs each, one launch, each doc against its own query.
--workload shared times 8 queries of 32 rows against the same 80,000 docs
(maxsim_rerank_multi, one call: plan, then per pass of 128 query rows a score and a
combine launch); its events bracket the whole call, and a doc token counts once per
query that scores it. --workload large_fp8 times the large workload with docs stored as
FP8 E4M3 bytes (scale 2^-8; maxsim_plan, maxsim_score_fp8, maxsim_finish_fp8), and
--workload shared_fp8 the shared workload with FP8 docs (maxsim_rerank_multi_fp8).

After the timed steps, unless --no-read-probe, the doc tensor is read once more by a
plain streaming read kernel (libmaxsim_probe.so, LDS-DMA and register loads) and the
rates are reported as read_ceiling: the read bandwidth this device actually sustains,
next to the published 8 TB/s that roofline.peak uses.

Cache eviction (flushed): after the K back-to-back steps that give `value`, each of
--flush-reps further steps runs right after a 1 GiB write that evicts the 256 MB MALL
and the L2s (outside the events); the write also keeps the GPU busy while the host
enqueues the step, so these events time the step's kernels and the gaps between them,
not the host's launch cost. `flushed` reports their median, p10 and p90, and those of
the score kernel alone.

--one-shot also times the one-shot entry point (maxsim_rerank, maxsim_rerank_fp8 or
maxsim_rerank_pairs) with a synchronise after every call, host wall clock per call,
against the staged path (plan, score, finish on a caller workspace) timed the same way.
--path one-shot makes the one-shot call itself the timed step (events around the call):
for one query of at most 8192 docs the self-scheduling range kernel and its combine.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload large]
                    [--no-cpu-baseline] [--no-read-probe] [--copy-probe]
                    [--flush-reps N] [--one-shot] [--path staged|one-shot]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16
METRIC = "doc tokens scored/sec and achieved HBM GB/s (% of peak), MaxSim rerank, 1 GPU"
SCORE_SOURCES = [
    os.path.join(ROOT, "late_interaction_reranking_amd", "csrc", f)
    for f in ("maxsim_score.h", "maxsim_score_inst.hip", "maxsim_common.h", "maxsim_sched.h")
]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def score_source_digest() -> str:
    h = hashlib.sha256()
    for p in SCORE_SOURCES:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per score launch from committed rocprofv3 counter runs, if they were
    taken on the current score-kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("score_source_digest") != score_source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


PROBE_LIBRARY = os.path.join(ROOT, "late_interaction_reranking_amd", "libmaxsim_probe.so")


def read_ceiling(buf, reps: int = 5):
    """The device's plain streaming read rate over `buf` (the doc tensor, already in HBM):
    libmaxsim_probe.so reads it once per launch with LDS-DMA loads (the score kernel's
    tile path, nothing consumed) and with register loads; GB/s from HIP events around
    each launch on torch's current stream, averaged over `reps` launches after one
    warm-up."""
    import ctypes

    import torch  # before the library: it must bind to torch's HIP runtime (same soname)

    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.maxsim_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    blocks = int(lib.maxsim_probe_blocks())
    if blocks < 1:
        raise RuntimeError("maxsim_probe_blocks failed")
    base = buf if buf._base is None else buf._base
    nbytes = base.numel() * base.element_size()
    nbytes -= nbytes % 16
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=base.device)
    stream = torch.cuda.current_stream().cuda_stream
    out = {"kernel": "libmaxsim_probe.so: probe_lds_kernel, probe_reg_kernel", "bytes": nbytes,
           "blocks": blocks, "launches": reps}
    for mode, key in ((0, "lds_dma_GBps"), (1, "register_GBps")):
        ms = []
        for i in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = lib.maxsim_probe_read(base.data_ptr(), nbytes, mode, blocks, sink.data_ptr(), stream)
            b.record()
            if rc != 0:
                raise RuntimeError(f"maxsim_probe_read returned {rc}")
            torch.cuda.synchronize()
            if i > 0:
                ms.append(a.elapsed_time(b))
        out[key] = nbytes / (sum(ms) / len(ms) * 1e-3) / 1e9
    return out


def algorithmic_bytes(w) -> int:
    """Doc rows read once (2 d bytes per doc token, d with FP8 docs), 8 B of offset/length and 4 B of
    score per doc, and the query rows once; a multi-query batch adds each doc's 4 B
    query index and 8 B of offset/length per query; queries sharing the docs write
    4 B of score per (query, doc)."""
    q_bytes = w.Q.shape[0] * w.d * 2
    if w.shared_docs:
        return w.doc_bytes + w.B * (8 + 4 * w.nq) + q_bytes
    if w.multi_query:
        return w.doc_bytes + w.B * 16 + q_bytes + w.nq * 8
    return w.doc_bytes + w.B * 12 + q_bytes


def algorithmic_flops(w) -> float:
    """2 d multiply-adds per (query row, doc token) pair."""
    if w.shared_docs:
        return 2.0 * w.d * float(w.q_lengths.astype(int).sum()) * w.doc_tokens
    if w.multi_query:
        import numpy as np

        ql = w.q_lengths[w.doc_query].astype(np.int64)
        return 2.0 * w.d * float(np.dot(ql, w.lengths.astype(np.int64)))
    return 2.0 * w.Lq * w.d * w.doc_tokens


def score_launches(w) -> int:
    """Score launches of one maxsim_rerank_multi call: queries are packed in order into
    passes of at most one register group of 16-row query tiles (min(32 // ceil(d / 32), 8)
    tiles), a longer query alone; 1 for the other workload forms."""
    if not w.shared_docs:
        return 1
    group = min(32 // -(-w.d // 32), 8)
    passes, cur = 0, 0
    for L in (int(x) for x in w.q_lengths):
        t = -(-L // 16)
        if t == 0:
            continue
        if cur and cur + t > group:
            passes, cur = passes + 1, 0
        cur += t
        if cur >= group:
            passes, cur = passes + 1, 0
    return passes + (1 if cur else 0)


def cpu_info() -> dict:
    """The host CPU as /proc/cpuinfo names it (the full model string, vendor, family,
    model, logical CPUs listed) and the CPUs this process may run on."""
    info = {"model_name": "unknown"}
    try:
        with open("/proc/cpuinfo") as fh:
            text = fh.read()
        first = text.split("\n\n", 1)[0]
        for line in first.splitlines():
            if ":" not in line:
                continue
            k, v = (x.strip() for x in line.split(":", 1))
            if k == "model name":
                info["model_name"] = v
            elif k in ("vendor_id", "cpu family", "model", "stepping", "cpu MHz", "cache size"):
                info[k.replace(" ", "_")] = v
        info["logical_cpus_listed"] = text.count("processor\t:")
    except OSError:
        pass
    info["affinity_cpus"] = len(os.sched_getaffinity(0))
    info["os_cpu_count"] = os.cpu_count()
    quota = cgroup_cpu_quota()
    if quota is not None:
        info["cgroup_cpu_quota"] = quota
    if os.environ.get("OMP_NUM_THREADS"):
        info["OMP_NUM_THREADS"] = os.environ["OMP_NUM_THREADS"]
    return info


def cgroup_cpu_quota():
    """CPUs' worth of time the process's cgroup may use (cgroup v2 cpu.max), or None."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            quota, period = fh.read().split()[:2]
        if quota == "max":
            return None
        return float(quota) / float(period)
    except (OSError, ValueError):
        return None


def host_threads() -> int:
    """Threads for the oracle: every CPU this process may run on (its affinity mask),
    but no more than its CPU share where one is set (a cgroup quota, or the machine's
    OMP_NUM_THREADS): threads beyond the share would only queue for the same time."""
    n = len(os.sched_getaffinity(0))
    quota = cgroup_cpu_quota()
    if quota is not None:
        n = min(n, max(1, int(quota)))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle, unchanged, on the host cores: whole docs in doc order until the time
    budget is spent (or all docs are done). Returns the record and the oracle's scores
    of the docs it scored (doc ids 0 .. n-1)."""
    import numpy as np

    import oracle

    threads = host_threads()
    oracle.maxsim_workload(w, docs=np.arange(min(8, w.B)), threads=threads)  # load + warm
    done_docs = 0
    tokens = 0
    parts = []
    t0 = time.perf_counter()
    batch = 256
    while done_docs < w.B and time.perf_counter() - t0 < budget_s:
        ids = np.arange(done_docs, min(w.B, done_docs + batch))
        parts.append(oracle.maxsim_workload(w, docs=ids, threads=threads))
        tokens += int(w.lengths[ids].astype(np.int64).sum()) * (w.nq if w.shared_docs else 1)
        done_docs += len(ids)
        batch = min(batch * 2, 8192)
    dt = time.perf_counter() - t0
    rec = {
        "value": tokens / dt,
        "unit": "doc tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {done_docs} of {w.B} docs ({tokens} doc tokens"
                  + (f" summed over {w.nq} queries" if w.shared_docs else "")
                  + f") of the same workload, fp64 oracle, {dt:.1f} s wall",
        "cpu_model": cpu_info()["model_name"],
        "cpu": cpu_info(),
    }
    if w.shared_docs:
        return rec, (np.concatenate(parts, axis=1) if parts else np.zeros((w.nq, 0)))
    return rec, (np.concatenate(parts) if parts else np.zeros(0))


def _top10_ok(g, ref) -> bool:
    """The GPU's top-10 (ties by lower index), scored by the oracle, reproduces the
    oracle's sorted top-10 rank by rank within the tolerance."""
    import numpy as np

    n = len(ref)
    order_ref = np.lexsort((np.arange(n), -ref))[:10]
    order_gpu = np.lexsort((np.arange(n), -g))[:10]
    want = ref[order_ref]
    mine = ref[order_gpu]
    return bool(np.all(np.abs(mine - want) <= 1e-3 * (1 + np.abs(want))))


def parity_summary(gpu, ref, w):
    """Scores of the timed run against the oracle (docs 0 .. n-1 that the CPU baseline
    scored), under the acceptance rule |gpu - oracle| <= 1e-3 (1 + |oracle|). The top-10
    check needs every doc of a ranking scored: the whole batch for one query (or for
    each query sharing the docs), else each query of a pairs batch whose docs were all
    checked."""
    import numpy as np

    if w.shared_docs:
        # ref: [nq, n]
        n = ref.shape[1]
        g = np.asarray(gpu, np.float64)[:, :n]
        inf = np.isinf(ref)
        err = np.abs(g[~inf] - ref[~inf]) / (1.0 + np.abs(ref[~inf]))
        out = {"docs_checked": int(n), "queries": int(ref.shape[0]),
               "max_scaled_err": float(err.max()) if err.size else 0.0,
               "violations": int(np.sum(~(err <= 1e-3))) + int(np.sum(g[inf] != ref[inf])),
               "top10_ok": None}
        if n == w.B:
            out["top10_ok"] = bool(all(_top10_ok(g[j], ref[j]) for j in range(ref.shape[0])))
        return out
    n = len(ref)
    g = np.asarray(gpu[:n], np.float64)
    inf = np.isinf(ref)
    fin = ~inf
    err = np.abs(g[fin] - ref[fin]) / (1.0 + np.abs(ref[fin]))
    bad = int(np.sum(~(err <= 1e-3))) + int(np.sum(g[inf] != ref[inf]))
    out = {"docs_checked": int(n), "max_scaled_err": float(err.max()) if err.size else 0.0,
           "violations": bad, "top10_ok": None}
    if not w.multi_query:
        if n == w.B:
            out["top10_ok"] = _top10_ok(g, ref)
        return out
    dq = w.doc_query
    done = [j for j in np.unique(dq[:n]) if not np.any(dq[n:] == j)]
    oks = [_top10_ok(g[dq[:n] == j], ref[dq[:n] == j]) for j in done if np.sum(dq[:n] == j) >= 10]
    if oks:
        out["top10_ok"] = bool(all(oks))
        out["top10_queries_checked"] = len(oks)
    return out


def percentiles(ms) -> dict:
    """median, p10, p90, mean, min and max of a list of times."""
    import numpy as np

    a = np.asarray(ms, np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "min": float(a.min()),
            "max": float(a.max()), "n": int(a.size)}


def time_one_shot(w, lir, Q, X, offs, lens, scores, ws, step, dev, args):
    """Host wall time per call of the one-shot entry point with a synchronise after each
    call, against the staged step (plan, score, finish on the caller's workspace) timed
    the same way; reps alternate between the two."""
    import torch

    if w.shared_docs:
        return None
    if w.multi_query:
        qo, ql, dq = (torch.from_numpy(a).to(dev) for a in (w.q_offsets, w.q_lengths, w.doc_query))

        def call():
            lir.rerank_pairs(Q, qo, ql, w.Lq, X, offs, lens, dq, scores=scores)
    elif w.X8 is not None:
        def call():
            lir.maxsim_rerank_fp8(Q, X, offs, lens, w.doc_scale, scores=scores)
    else:
        def call():
            lir.rerank(Q, X, offs, lens, scores=scores)
    reps = 200 if w.doc_bytes < 1e9 else 20
    for _ in range(5):
        call()
        step()
    torch.cuda.synchronize()
    one, staged = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        one.append((t1 - t0) * 1e6)
        staged.append((t2 - t1) * 1e6)
    a, b = percentiles(one), percentiles(staged)
    name = ("maxsim_rerank_pairs" if w.multi_query else
            "maxsim_rerank_fp8" if w.X8 is not None else "maxsim_rerank")
    return {"entry": name, "reps": reps, "call_us": a, "staged_us": b,
            "ratio_median": a["median"] / b["median"]}


def fp8_quality(gpu, w):
    """How far FP8 E4M3 storage moves scores and rankings: the GPU's FP8 scores against
    the fp16 oracle over the same docs before quantisation (all docs)."""
    import numpy as np

    import oracle

    ref = oracle.maxsim(w.dtype, w.Q, w.X, w.offsets, w.lengths, d=w.d, threads=host_threads())
    err = np.abs(gpu - ref) / (1.0 + np.abs(ref))
    n = len(ref)
    rank_ref = np.empty(n, np.int64)
    rank_gpu = np.empty(n, np.int64)
    order_ref = np.lexsort((np.arange(n), -ref))
    order_gpu = np.lexsort((np.arange(n), -gpu))
    rank_ref[order_ref] = np.arange(n)
    rank_gpu[order_gpu] = np.arange(n)
    out = {"docs": int(n), "reference": "fp16 oracle on the unquantised docs",
           "max_scaled_err": float(err.max()), "median_scaled_err": float(np.median(err)),
           "docs_outside_1e-3": int(np.sum(err > 1e-3))}
    for k in (10, 100):
        top_ref, top_gpu = order_ref[:k], order_gpu[:k]
        out[f"top{k}_overlap"] = int(len(set(top_ref.tolist()) & set(top_gpu.tolist())))
        out[f"top{k}_max_rank_displacement"] = int(np.max(np.abs(rank_gpu[top_ref] - rank_ref[top_ref])))
    # Spearman rank correlation over all docs
    out["spearman"] = float(1.0 - 6.0 * np.sum((rank_gpu - rank_ref).astype(np.float64) ** 2)
                            / (n * (n * n - 1.0)))
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large",
                    choices=["tiny", "colbert", "long_doc", "scattered", "large", "pairs", "shared",
                             "large_fp8", "shared_fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--topk", type=int, default=0,
                    help="also select the k best docs on the GPU in every step (maxsim_topk)")
    ap.add_argument("--short", action="store_true",
                    help="single-query workloads: one launch per step, one workgroup per doc "
                         "(maxsim_rerank_short) instead of plan + score + combine")
    ap.add_argument("--path", choices=["staged", "one-shot"], default="staged",
                    help="single-query workloads: 'staged' times maxsim_plan, maxsim_score and "
                         "maxsim_finish on a caller workspace (events around the score kernel); "
                         "'one-shot' times maxsim_rerank (maxsim_rerank_fp8) itself, events around the "
                         "whole call: for at most 8192 docs the self-scheduling range kernel and its "
                         "combine, else plan, score and combine")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one step captured in a HIP graph (no host "
                         "launch cost per kernel); the per-launch roofline still comes from eager steps")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the read-ceiling probe (a plain streaming read of the doc tensor, "
                         "reported as read_ceiling)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one plain 2 GiB device copy (counter calibration)")
    ap.add_argument("--flush-reps", type=int, default=None,
                    help="steps timed one by one after a 1 GiB cache-evicting write (default: 200 "
                         "for workloads under 100 MB of doc rows, 50 under 1 GB, else 20; 0: none)")
    ap.add_argument("--one-shot", action="store_true",
                    help="also time the one-shot entry point with a synchronise after every call, "
                         "against the staged path timed the same way")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(docs would be sharded across GPUs by the caller); use --gpus 1",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import late_interaction_reranking_amd as lir
    import workloads

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    lir.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    log(f"generating workload {args.workload}")
    t0 = time.perf_counter()
    if args.workload == "large_fp8" and not args.no_cpu_baseline:
        # keep the 16-bit docs: the FP8 scores are also compared with the fp16 oracle
        w = workloads.to_fp8(workloads.large(), keep_x=True)
        w.name = "large_fp8"
    else:
        w = workloads.make(args.workload)
    log(f"generated B={w.B} rows={w.T} doc tokens={w.doc_tokens} in {time.perf_counter() - t0:.1f} s")
    tdt = torch.float16 if w.dtype == "f16" else torch.bfloat16
    Q = torch.from_numpy(w.Q.view(np.int16)).to(dev).view(tdt)
    if w.X8 is not None:
        X = torch.from_numpy(w.X8).to(dev)[:, : w.d]
    else:
        X = torch.from_numpy(w.X.view(np.int16)).to(dev).view(tdt)[:, : w.d]
    offs = torch.from_numpy(w.offsets).to(dev)
    lens = torch.from_numpy(w.lengths).to(dev)
    scores = torch.empty(w.B, dtype=torch.float32, device=dev)
    ws = torch.empty(lir.maxsim_workspace_size(w.Lq, w.d, w.B), dtype=torch.uint8, device=dev)
    if w.shared_docs:
        scores = torch.empty((w.nq, w.B), dtype=torch.float32, device=dev)
        q_lengths = [int(x) for x in w.q_lengths]

        def plan():
            pass
    elif w.multi_query:
        qo, ql, dq = (torch.from_numpy(a).to(dev) for a in (w.q_offsets, w.q_lengths, w.doc_query))

        def plan():
            lir.maxsim_plan_pairs(offs, lens, dq, qo, ql, w.Q.shape[0], w.Lq, w.d, ws)
    else:
        def plan():
            lir.maxsim_plan(offs, lens, w.Lq, w.d, ws)
    if args.short and (w.shared_docs or w.multi_query or args.topk):
        print("--short applies to single-query workloads without --topk", file=sys.stderr)
        return 2
    one_shot_path = args.path == "one-shot"
    if one_shot_path and (w.shared_docs or w.multi_query or args.topk or args.short):
        print("--path one-shot applies to single-query workloads without --topk or --short", file=sys.stderr)
        return 2
    if args.topk:
        if w.shared_docs or w.multi_query:
            print("--topk applies to single-query workloads", file=sys.stderr)
            return 2
        import ctypes

        nb = ctypes.c_size_t(0)
        lir.load().maxsim_topk_workspace_size(w.B, args.topk, ctypes.byref(nb))
        tk_ws = torch.empty(int(nb.value), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("uploaded")
    tk_events = []

    def step(ev_a=None, ev_b=None, force_staged=False):
        if w.shared_docs:
            if ev_a is not None:
                ev_a.record()
            if w.X8 is not None:
                lir.maxsim_rerank_multi_fp8(Q, q_lengths, X, offs, lens, w.doc_scale, scores=scores)
            else:
                lir.rerank_multi(Q, q_lengths, X, offs, lens, scores=scores)
            if ev_b is not None:
                ev_b.record()
            return
        if one_shot_path and not force_staged:
            if ev_a is not None:
                ev_a.record()
            if w.X8 is not None:
                lir.maxsim_rerank_fp8(Q, X, offs, lens, w.doc_scale, scores=scores)
            else:
                lir.rerank(Q, X, offs, lens, scores=scores)
            if ev_b is not None:
                ev_b.record()
            return
        if args.short:
            if ev_a is not None:
                ev_a.record()
            if w.X8 is not None:
                lir.maxsim_rerank_short_fp8(Q, X, offs, lens, w.doc_scale, scores=scores)
            else:
                lir.maxsim_rerank_short(Q, X, offs, lens, scores=scores)
            if ev_b is not None:
                ev_b.record()
            return
        plan()
        if ev_a is not None:
            ev_a.record()
        if w.X8 is not None:
            lir.maxsim_score_fp8(Q, X, offs, lens, w.doc_scale, ws, scores=scores)
        else:
            lir.maxsim_score(Q, X, offs, lens, ws, scores=scores, Lq=w.Lq)
        if ev_b is not None:
            ev_b.record()
        if w.X8 is not None:
            lir.maxsim_finish_fp8(Q, w.B, w.doc_scale, ws, scores)
        else:
            lir.maxsim_finish(Q, w.B, ws, scores, Lq=w.Lq)
        if args.topk:
            if ev_a is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            lir.maxsim_topk(scores, args.topk, tk_ws)
            if ev_a is not None:
                e1.record()
                tk_events.append((e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for a, b in evs:
        step(a, b)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    score_ms = [a.elapsed_time(b) for a, b in evs]
    score_avg_ms = sum(score_ms) / len(score_ms)
    # Step periods: from one step's score-kernel start to the next one's (the last to the end).
    step_ms = [evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(args.steps - 1)]
    step_ms.append(evs[-1][0].elapsed_time(end))
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step, score kernel {score_avg_ms:.4f} ms avg "
        f"(min {min(score_ms):.4f}, max {max(score_ms):.4f})")

    # Flushed: each step right after a 1 GiB write (its own events bracket the step only).
    flush_reps = args.flush_reps
    if flush_reps is None:
        flush_reps = 200 if w.doc_bytes < 100e6 else (50 if w.doc_bytes < 1e9 else 20)
    flushed = None
    if flush_reps > 0:
        # Two passes, so that each timed interval holds as few event markers as possible
        # (a marker costs microseconds of GPU time): the whole step, then (staged path)
        # the score kernel alone. After each evicting write an untimed marker comes first,
        # so that the write's completion is not charged to the step.
        evict = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        pad = torch.cuda.Event()
        fl = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(flush_reps)]
        torch.cuda.synchronize()
        for i, (s0, s1) in enumerate(fl):
            evict.fill_(i & 255)
            pad.record()
            s0.record()
            step()
            s1.record()
        torch.cuda.synchronize()
        f_step = [s0.elapsed_time(s1) for s0, s1 in fl]
        if one_shot_path or args.short or w.shared_docs:
            f_score = f_step  # the step is one call, bracketed by the same events
        else:
            for i, (a, b) in enumerate(fl):
                evict.fill_(i & 255)
                pad.record()
                step(a, b)
            torch.cuda.synchronize()
            f_score = [a.elapsed_time(b) for a, b in fl]
        del evict
        flushed = {"reps": flush_reps, "evict_bytes": 1 << 30,
                   "step_ms": percentiles(f_step), "score_ms": percentiles(f_score)}
        log(f"flushed {flush_reps} steps: step median {flushed['step_ms']['median']:.4f} ms, "
            f"score kernel median {flushed['score_ms']['median']:.4f} ms")

    ms_per_step_eager = ms_per_step
    if args.graph:
        # One whole step (every launch of it) captured once and replayed: the inputs stay
        # where they are, and every replay redoes all of the step's work.
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(end) / args.steps
        log(f"timed {args.steps} graph replays: {ms_per_step:.4f} ms/step (eager {ms_per_step_eager:.4f})")

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: one device copy of 2 GiB (reads 2 GiB, writes 2 GiB)")
        del src, dst

    one_shot = None
    if args.one_shot:
        one_shot = time_one_shot(w, lir, Q, X, offs, lens, scores, ws, lambda: step(force_staged=True), dev, args)
        log(f"one-shot: {one_shot['call_us']['median']:.1f} us per synced call, staged "
            f"{one_shot['staged_us']['median']:.1f} us (ratio {one_shot['ratio_median']:.2f})")

    ceiling = None
    if not args.no_read_probe:
        ceiling = read_ceiling(X)
        log(f"read ceiling over {ceiling['bytes']} bytes: LDS-DMA {ceiling['lds_dma_GBps']:.0f} GB/s, "
            f"registers {ceiling['register_GBps']:.0f} GB/s")

    alg_bytes = algorithmic_bytes(w)
    launches = score_launches(w)
    # Per score launch: one maxsim_rerank_multi call holds `launches` score launches, each
    # reading the docs once (its events bracket the whole call, plan and combines too).
    launch_bytes = alg_bytes if launches == 1 else w.doc_bytes + w.B * (8 + 4 * w.nq // launches) + (
        w.Q.shape[0] * w.d * 2 // launches)
    launch_ms = score_avg_ms / launches
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
    flops = algorithmic_flops(w)
    scored_tokens = w.doc_tokens * (w.nq if w.shared_docs else 1)
    tokens_per_s = scored_tokens / (ms_per_step * 1e-3)
    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "doc tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 docs, " if w.X8 is not None else "") + ("f16" if w.dtype == "f16" else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: " + (f"{w.nq} queries of up to " if w.multi_query else "")
                        + f"Lq={w.Lq} d={w.d} B={w.B} {w.dtype}, "
                        f"{w.doc_tokens} doc tokens in a [{w.T}, {w.X8.shape[1] if w.X8 is not None else w.stride}] "
                        + ("FP8 E4M3 (scale %g) " % w.doc_scale if w.X8 is not None else "")
                        + f"tensor, seed {w.seed}",
            "Lq": w.Lq, "d": w.d, "B": w.B, "doc_tokens": w.doc_tokens, "rows": w.T,
            "queries": w.nq,
            "parallelism": "1 GPU",
        },
        "launch": ("HIP graph replay of one captured step" if args.graph
                   else "eager: one host launch per kernel"),
        "path": ("one launch, one workgroup per doc (maxsim_rerank_short)" if args.short
                 else (("one-shot maxsim_rerank: self-scheduling range kernel + combine" if w.B <= 8192
                        else "one-shot maxsim_rerank: plan, score, combine") if one_shot_path
                       else "scheduled: plan, score, combine")),
        "ms_per_step_eager": ms_per_step_eager,
        "value_counts": ("each (query, doc token) pair once" if w.shared_docs else "each doc token once"),
        "hbm_GBps_step": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "pct_of_hbm_peak_step": 100.0 * alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "mfma_util_algorithmic": flops / (score_avg_ms * 1e-3) / (MFMA_F16_PEAK_TFLOPS * 1e12),
        "roofline": {
            "bound": "hbm",
            "kernel": ("score_kernel (per pass: the maxsim_rerank_multi call's time, plan and combines "
                       "included, over its score launches)" if w.shared_docs
                       else ("short_kernel" if args.short else
                             ("whole maxsim_rerank call (every kernel of the step)" if one_shot_path
                              else "score_kernel"))),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None if (args.short or one_shot_path) else measured_traffic(w.name),
            "algorithmic_bytes_per_launch": launch_bytes,
            "avg_launch_ms": launch_ms,
            "launches_per_step": launches,
        },
        "step_ms": percentiles(step_ms),
        "score_ms": percentiles(score_ms),
        "flushed": flushed,
        "cpu_baseline": None,
        "parity": None,
    }
    if one_shot is not None:
        rec["one_shot"] = one_shot
    if ceiling is not None:
        ceiling["score_frac_of_ceiling"] = achieved / max(ceiling["lds_dma_GBps"], ceiling["register_GBps"])
        rec["read_ceiling"] = ceiling
    if args.topk:
        tk_ms = [a.elapsed_time(b) for a, b in tk_events[: args.steps]]
        rec["topk"] = {"k": args.topk, "avg_ms": sum(tk_ms) / len(tk_ms), "included_in_step": True}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"], ref = cpu_baseline(w)
        rec["parity"] = parity_summary(scores.cpu().numpy(), ref, w)
        if w.X8 is not None and not w.shared_docs and w.X.shape[0] == w.T:
            log("fp8 quality: fp16 oracle on the unquantised docs")
            rec["fp8_quality"] = fp8_quality(scores.cpu().numpy().astype(np.float64), w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
