"""Benchmark: one CP rank's share of zigzag prefill attention on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  1. host zigzag metadata (cp_meta_build) and its one host->device copy,
  2. KV scatter of the all-gathered K and V into the paged pool,
  3. zigzag rerange of the gathered K and V back to token order,
  4. the fused causal attention of both zigzag halves.
Inputs are resident in HBM before the timed region starts.

Default workload: cp_size=8, one sequence of 131072 tokens (blocks of 8192),
rank 3 (blocks 3 and 12; kv_len 32768 and 106496), H_q=64, H_kv=8, D=128,
paged KV with page size 64 and permuted pages, bf16.

``--workload`` picks any other synthetic workload.  For the AllGather-KV
shares (local Q against the ordered global K/V, whose pad suffix is never
read) a step is the host metadata, its copy and the non-causal attention
launch; ``--rank`` picks the rank's slice, ``--kv-heads`` the KV head
count and ``--q-heads`` the query head count (the Ulysses head share).

Prints one JSON line.  ``value`` is useful attention TFLOP/s over the whole
step (masked-out pairs and skipped tiles are not counted).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def causal_pairs(q_len: int, kv_len: int) -> int:
    """(query, visible key) pairs of one causal bottom-right segment, closed form."""
    off = kv_len - q_len
    # sum_{i=0}^{q_len-1} (i + off + 1)
    return q_len * (off + 1) + q_len * (q_len - 1) // 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_cp8_s131072_r3")
    ap.add_argument("--rank", type=int, default=None, help="CP rank (zigzag) or AllGather-KV rank")
    ap.add_argument("--kv-heads", type=int, default=None, help="KV heads (AllGather-KV workloads)")
    ap.add_argument("--q-heads", type=int, default=None,
                    help="query heads (AllGather-KV workloads; e.g. the share a Ulysses group leaves on one GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768, help="query rows in the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing attention on the other workload shapes")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic.json from rocprofv3 --pmc runs of FETCH_SIZE and WRITE_SIZE "
                         "(bench step, then --calibrate-copy) and exit")
    return ap.parse_args()


def calibrate_copy(steps: int) -> None:
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch.
    Profiler byte counters of this run scale the attention kernel's counters."""
    import torch
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 2, "calibrate_copy_bytes_written":
                      dst.numel() * 2, "launches": steps}))


def kernel_sha256(paths) -> str:
    """SHA-256 over a kernel's device sources, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")


def traffic_for(kernel: str, workload: str, rank: int):
    """Measured HBM bytes per launch of ``kernel`` (FETCH_SIZE and WRITE_SIZE
    counters scaled by the plain-copy calibration), if the committed record
    was taken on this exact kernel source, workload and rank; else None."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        recs = json.load(f)
    rec = recs.get("kernels", {}).get(kernel)
    if rec is None or recs.get("workload") != workload or recs.get("rank") != rank:
        return None
    if rec.get("kernel_sha256") != kernel_sha256(KERNEL_SRC[kernel]):
        return None
    return rec.get("bytes_per_launch")


def _counter_means(run_dir: str, counter: str):
    """Mean counter value (KiB) per dispatch, by kernel, from a rocprofv3
    --pmc run's counter_collection CSV under run_dir."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for i, row in enumerate(csv.DictReader(f)):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                key = next((k for k in KERNEL_SRC if k in name), "copy" if "copyBuffer" in name else None)
                if key is None:
                    continue
                disp = (fn, row.get("Dispatch_Id") or i)
                per.setdefault(key, {})
                per[key][disp] = per[key].get(disp, 0.0) + float(row["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def record_traffic(fetch_dir, write_dir, fetch_copy_dir, write_copy_dir, workload, rank):
    """Write profiles/traffic.json from four rocprofv3 --pmc runs: FETCH_SIZE
    and WRITE_SIZE of the bench step, and of --calibrate-copy (1 GiB read +
    1 GiB written per launch), which gives the scale of each counter."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cf, cw = _counter_means(fetch_copy_dir, "FETCH_SIZE")["copy"], _counter_means(write_copy_dir, "WRITE_SIZE")["copy"]
    gib_kib = float(1 << 20)
    ff, wf = gib_kib / cf, gib_kib / cw
    out = {"workload": workload, "rank": rank,
           "copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "fetch_size_kib": cf,
                                "write_size_kib": cw, "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    for k in KERNEL_SRC:
        if k not in fetch or k not in write:
            continue
        out["kernels"][k] = {
            "kernel_sha256": kernel_sha256(KERNEL_SRC[k]),
            "fetch_size_kib_per_launch": fetch[k], "write_size_kib_per_launch": write[k],
            "bytes_per_launch": int(round((fetch[k] * ff + write[k] * wf) * 1024))}
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def oracle_threads() -> int:
    """BLAS threads the oracle's numpy runs on."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def oracle_blas() -> str:
    """BLAS library behind the oracle's numpy (name and version)."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return " ".join(filter(None, [blas[0].get("internal_api"), blas[0].get("version")])) if blas else "unknown"
    except Exception:
        return "unknown"


def cpu_baseline(w, meta_lists, q_loc, k_seq, v_seq, n_rows: int):
    """Time the fp64 oracle on an evenly spaced sample of query rows of the
    same rank share; scale to useful TFLOP/s."""
    import numpy as np
    from oracle import attention as oatt
    threads = oracle_threads()
    segs = meta_lists["segments"]
    per = max(1, n_rows // len(segs))
    scale = 1.0 / math.sqrt(w.d)
    q_cpu = q_loc.cpu()
    k64 = k_seq.to(dtype=__import__("torch").float64).numpy()
    v64 = v_seq.to(dtype=__import__("torch").float64).numpy()
    flops = 0
    t0 = time.perf_counter()
    for (r0, q_len, kv_len) in segs:
        loc = np.linspace(0, q_len - 1, per).astype(np.int64)
        oatt.attention_rows(q_cpu[(r0 + loc).tolist()], loc, k64, v64, q_len, kv_len, True, scale)
        off = kv_len - q_len
        flops += 4 * w.d * w.h_q * int(np.sum(loc + off + 1))
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "blas": oracle_blas(),
            "sample": f"{per * len(segs)} query rows ({per} evenly spaced per zigzag half) x {w.h_q} heads "
                      f"of the same rank share, all visible keys, numpy float64 in one process whose BLAS "
                      f"runs on `cores` threads; {dt:.1f} s"}


def cpu_baseline_copies(w, rank, lens, k_g, indptr, indices, n_pages):
    """Time the oracle's metadata (pure Python), its rerange and its KV
    scatter (numpy row copies) on K of the same share; GB/s as the device
    copies count them (each row read once and written once)."""
    import numpy as np
    from oracle import layout, zigzag_meta
    total = sum(lens)
    t0 = time.perf_counter()
    mo = zigzag_meta.build(w.cp_size, rank, total, extend_lens=lens)
    meta_s = time.perf_counter() - t0
    gathered = k_g.view(__import__("torch").int16).numpy()
    row_bytes = w.h_kv * w.d * 2
    t0 = time.perf_counter()
    layout.rerange(gathered, mo)
    rer_s = time.perf_counter() - t0
    pool = np.zeros((n_pages, w.page_size, w.h_kv, w.d), dtype=np.int16)
    t0 = time.perf_counter()
    layout.kv_scatter(gathered, mo, pool, indptr, indices, w.page_size)
    sc_s = time.perf_counter() - t0
    moved = 2 * total * row_bytes
    return {"meta_ms": round(meta_s * 1e3, 3), "rerange_gbps": round(moved / rer_s / 1e9, 2),
            "scatter_gbps": round(moved / sc_s / 1e9, 2), "cores": 1, "kind": "oracle",
            "sample": f"K of the same share ({total} rows of {row_bytes} B): zigzag_meta.build, "
                      f"layout.rerange and layout.kv_scatter; {meta_s + rer_s + sc_s:.1f} s"}


def cpu_baseline_allgather(w, h_q, q_loc, k_g, v_g, doc_cu, q_start, n_rows: int, packed: bool):
    """Time the fp64 oracle on evenly spaced local query rows of the
    AllGather-KV share; scale to useful TFLOP/s."""
    import numpy as np
    from oracle import attention as oatt
    threads = oracle_threads()
    n = q_loc.shape[0]
    rows = sorted(set(np.linspace(0, n - 1, n_rows).astype(np.int64).tolist()))
    scale = 1.0 / math.sqrt(w.d)
    t0 = time.perf_counter()
    if packed:
        oatt.allgather_kv_packed(q_loc, k_g, v_g, doc_cu, q_start, scale, rows=rows)
    else:
        q_real = max(0, min(n, doc_cu[-1] - q_start))
        oatt.allgather_kv(q_loc, k_g, v_g, q_real, doc_cu[-1], scale, rows=rows)
    dt = time.perf_counter() - t0
    visible = 0
    for r in rows:
        g = q_start + r
        for b in range(len(doc_cu) - 1):
            if doc_cu[b] <= g < doc_cu[b + 1]:
                visible += doc_cu[b + 1] - doc_cu[b]
    flops = 4 * w.d * h_q * visible
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "blas": oracle_blas(),
            "sample": f"{len(rows)} evenly spaced local query rows x {h_q} heads of the same share, "
                      f"all visible keys, numpy float64 in one process whose BLAS runs on `cores` threads; "
                      f"{dt:.1f} s"}


def run_timed(torch, step, names, warmup: int, steps: int):
    """Run ``warmup`` untimed steps, then ``steps`` timed ones.  step(ev)
    records ev[i] before phase names[i] and ev[-1] after the last phase (ev
    is None when untimed).  Every timed step has its own events, so the host
    prepares the next step while the GPU runs this one; the device is
    synchronised only around the timed region.  Returns (wall ms per step,
    {phase: mean ms}, {phase: [ms of every step]})."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    allocs0 = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    run_timed.allocations = torch.cuda.memory_stats().get("allocation.all.allocated", 0) - allocs0
    per = {n: [ev[i].elapsed_time(ev[i + 1]) for ev in evs] for i, n in enumerate(names)}
    return wall * 1e3 / steps, {n: sum(v) / steps for n, v in per.items()}, per


def result_line(args, useful_flops: float, ms_step: float, attn_ms: float, config: dict,
                traffic) -> dict:
    attn_tflops = useful_flops / (attn_ms * 1e-3) / 1e12
    return {
        "metric": "CP-rank prefill attn useful TFLOP/s (% MI355X bf16 MFMA peak); rerange GB/s",
        "value": round(useful_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "attn_ms": round(attn_ms, 4),
        "attn_ms_median": None,
        "attn_useful_tflops": round(attn_tflops, 2),
        "attn_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }


# each kernel's device code and the table layouts it reads
_CSRC = os.path.join(ROOT, "context_prefill_attention_amd", "csrc")
KERNEL_SRC = {
    "attn_kernel": [os.path.join(_CSRC, f) for f in ("cp_attn_kernel.h", "cp_internal.h")],
    "rerange_kernel": [os.path.join(_CSRC, f) for f in ("cp_copy.hip", "cp_internal.h")],
    "rerange_pair_kernel": [os.path.join(_CSRC, f) for f in ("cp_copy.hip", "cp_internal.h")],
    "scatter_kernel": [os.path.join(_CSRC, f) for f in ("cp_copy.hip", "cp_internal.h")],
}


def run_zigzag(args, w, torch, cpa, synth) -> dict:
    rank = w.ranks[0] if args.rank is None else args.rank
    dev = torch.device("cuda", 0)
    lens = synth.sequence_lengths(w)
    total = sum(lens)
    group = w.h_q // w.h_kv

    m0 = cpa.meta_build(w.cp_size, rank, lens, attn_group=group)
    n_loc, n_g = m0.n_local_rows, w.cp_size * m0.max_rank_len
    q_loc, k_g, v_g = synth.normal_bf16(w.seed, (n_loc, w.h_q, w.d), (n_g, w.h_kv, w.d), (n_g, w.h_kv, w.d))
    indptr, indices, n_pages = synth.page_table(w, lens)
    q_d, k_gd, v_gd = q_loc.to(dev), k_g.to(dev), v_g.to(dev)
    ip, ix = torch.from_numpy(indptr).to(dev), torch.from_numpy(indices).to(dev)
    k_pool = torch.zeros(n_pages, w.page_size, w.h_kv, w.d, dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros_like(k_pool)
    k_orig = torch.empty(total, w.h_kv, w.d, dtype=torch.bfloat16, device=dev)
    v_orig = torch.empty_like(k_orig)
    out = torch.empty_like(q_d)
    scale = 1.0 / math.sqrt(w.d)

    segs = [(m0.cu_seqlens_q_prev[b], m0.q_prev[b], m0.kv_len_prev[b]) for b in range(m0.bs)] + \
           [(m0.total_q_prev_tokens + m0.cu_seqlens_q_next[b], m0.q_next[b], m0.kv_len_next[b])
            for b in range(m0.bs)]
    pairs = sum(causal_pairs(q, kv) for (_r, q, kv) in segs)
    useful_flops = 4 * w.d * w.h_q * pairs
    row_bytes = w.h_kv * w.d * 2
    rerange_bytes = 2 * 2 * total * row_bytes      # K and V, each read once and written once
    scatter_bytes = 2 * 2 * total * row_bytes

    mbuf = cpa.MetaBuffers(dev)   # staging reused by every step: no allocation per build

    def step(ev):
        meta = cpa.meta_build(w.cp_size, rank, lens, attn_group=group, buffers=mbuf)
        if ev:
            ev[0].record()
        cpa.kv_scatter(meta, k_gd, v_gd, k_pool, v_pool, w.page_size, ip, ix)
        if ev:
            ev[1].record()
        cpa.zigzag_rerange_kv(meta, k_gd, k_orig, v_gd, v_orig, cpa.GATHERED_TO_ORIG)
        if ev:
            ev[2].record()
        cpa.prefill_attn(q_d, k_pool, v_pool, out, meta, scale, w.page_size, ip, ix)
        if ev:
            ev[3].record()

    ms_step, ph, per = run_timed(torch, step, ["scatter", "rerange", "attn"], args.warmup, args.steps)
    if not torch.isfinite(out).all():
        print("non-finite attention output", file=sys.stderr)
        sys.exit(1)
    config = {"workload": w.name, "cp_size": w.cp_size, "cp_rank": rank, "bs": len(lens),
              "seq_len": total, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
              "page_size": w.page_size, "parallelism": "one CP rank's share on one GPU"}
    res = result_line(args, useful_flops, ms_step, ph["attn"], config,
                      traffic_for("attn_kernel", w.name, rank))
    res["attn_ms_median"] = round(float(sorted(per["attn"])[len(per["attn"]) // 2]), 4)
    res["torch_allocations_in_timed_steps"] = run_timed.allocations
    roofline = res.pop("roofline")
    rer_t, sc_t = traffic_for("rerange_pair_kernel", w.name, rank), traffic_for("scatter_kernel", w.name, rank)
    res.update({
        "rerange_kv_ms": round(ph["rerange"], 4),
        "rerange_gbps": round(rerange_bytes / (ph["rerange"] * 1e-3) / 1e9, 1),
        "rerange_frac_of_hbm_peak": round(rerange_bytes / (ph["rerange"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        # one rerange launch moves K and V: algorithmic bytes vs the counters
        "rerange_bytes_per_launch": {"algorithmic": rerange_bytes, "counters": rer_t},
        "scatter_kv_ms": round(ph["scatter"], 4),
        "scatter_gbps": round(scatter_bytes / (ph["scatter"] * 1e-3) / 1e9, 1),
        "scatter_frac_of_hbm_peak": round(scatter_bytes / (ph["scatter"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "scatter_bytes_per_launch": {"algorithmic": scatter_bytes, "counters": sc_t},
        "roofline": roofline,
    })
    if not args.no_cpu_baseline:
        # the oracle reads synthetic token-order K/V of the same shape (its
        # timing does not depend on the values)
        res["cpu_baseline"] = cpu_baseline(w, {"segments": segs}, q_loc, k_g[:total], v_g[:total],
                                           args.cpu_rows)
        res["cpu_baseline_copies"] = cpu_baseline_copies(w, rank, lens, k_g, indptr, indices, n_pages)
    return res


def run_allgather(args, w, torch, cpa, synth) -> dict:
    rank = w.ag_rank if args.rank is None else args.rank
    h_kv = w.h_kv if args.kv_heads is None else args.kv_heads
    h_q = w.h_q if args.q_heads is None else args.q_heads
    if not 0 <= rank < w.ag_degree or h_kv < 1 or h_q < 1 or h_q % h_kv != 0:
        print(f"bad --rank {rank} (0..{w.ag_degree - 1}), --q-heads {h_q} or --kv-heads {h_kv} "
              f"(a divisor of the query heads)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    packed = w.packed_docs is not None
    share = w.kv_total // w.ag_degree
    q_start = rank * share
    doc_cu = synth.packed_doc_cu(w) if packed else [0, w.kv_real]
    q_real = max(0, min(share, w.kv_real - q_start))
    group = h_q // h_kv

    def build(buffers):
        if packed:
            return cpa.allgather_packed_meta_build(doc_cu, q_start, share, group, buffers=buffers)
        return cpa.allgather_meta_build(share, q_real, w.kv_real, group, buffers=buffers)

    qg, k_g, v_g = synth.normal_bf16(w.seed, (w.kv_total, h_q, w.d), (w.kv_total, h_kv, w.d),
                                     (w.kv_total, h_kv, w.d))
    k_g[w.kv_real:] = float("nan")     # the pad suffix must never be read
    v_g[w.kv_real:] = float("nan")
    q_loc = qg[q_start:q_start + share].contiguous()
    n_pages = w.kv_total // w.page_size
    q_d = q_loc.to(dev)
    k_pool = k_g.to(dev).view(n_pages, w.page_size, h_kv, w.d)   # contiguous K/V: identity table
    v_pool = v_g.to(dev).view(n_pages, w.page_size, h_kv, w.d)
    ip = torch.tensor([0, n_pages], dtype=torch.int32, device=dev)
    ix = torch.arange(n_pages, dtype=torch.int32, device=dev)
    out = torch.empty_like(q_d)
    scale = 1.0 / math.sqrt(w.d)
    pairs = sum(max(0, min(doc_cu[b + 1], q_start + share) - max(doc_cu[b], q_start)) *
                (doc_cu[b + 1] - doc_cu[b]) for b in range(len(doc_cu) - 1))
    useful_flops = 4 * w.d * h_q * pairs

    mbuf = cpa.MetaBuffers(dev)

    def step(ev):
        meta = build(mbuf)
        if ev:
            ev[0].record()
        cpa.prefill_attn(q_d, k_pool, v_pool, out, meta, scale, w.page_size, ip, ix)
        if ev:
            ev[1].record()

    ms_step, ph, per = run_timed(torch, step, ["attn"], args.warmup, args.steps)
    if not torch.isfinite(out).all():
        print("non-finite attention output", file=sys.stderr)
        sys.exit(1)
    config = {"workload": w.name, "ag_degree": w.ag_degree, "ag_rank": rank, "q_rows": share,
              "kv_total": w.kv_total, "kv_real": w.kv_real, "n_docs": len(doc_cu) - 1,
              "h_q": h_q, "h_kv": h_kv, "head_dim": w.d, "page_size": w.page_size,
              "parallelism": "one AllGather-KV rank's share on one GPU"}
    res = result_line(args, useful_flops, ms_step, ph["attn"], config,
                      traffic_for("attn_kernel", w.name, rank))
    res["attn_ms_median"] = round(float(sorted(per["attn"])[len(per["attn"]) // 2]), 4)
    res["torch_allocations_in_timed_steps"] = run_timed.allocations
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_allgather(w, h_q, q_loc, k_g, v_g, doc_cu, q_start,
                                                     args.cpu_rows, packed)
    return res


def time_launches(torch, launch, warmup: int, iters: int) -> float:
    """Mean ms per launch over ``iters`` back-to-back launches (HIP events on
    the current stream, after ``warmup`` untimed ones)."""
    for _ in range(warmup):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        launch()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


# Attention on the other workload shapes: (workload, rank, H_kv override or
# None, cached-prefix lengths or None).  The prefix share is the cached
# prefix + extend case: cp 4, a 4096-token prefix ahead of an 8192-token
# extend, next to a 6144-token sequence without prefix, pages of 64.
OTHER_CONFIGS = (
    [("tiny_cp2_s256", r, None) for r in (0, 1)]
    + [("gqa_cp2_s8192", r, None) for r in (0, 1)]
    + [("varlen_cp4_bs8", r, None) for r in range(4)]
    + [("allgather_kv_s32768", 1, h) for h in (8, 1)]
    + [("allgather_packed_s32768", r, 8) for r in (1, 3)]
    + [("prefix_cp4_p4096_e8192", r, None) for r in range(4)]
)
PREFIX_SHARE = {"extend": [8192, 6144], "prefix": [4096, 0], "cp_size": 4, "h_q": 32, "h_kv": 4,
                "d": 128, "page_size": 64, "seed": 41}


def other_configs(torch, cpa, synth) -> list:
    """Time cp_prefill_attn alone on every other workload shape.  Inputs are
    seeded N(0,1) bf16 drawn on the device (their values do not change the
    work); page tables and metadata are the workloads' own."""
    dev = torch.device("cuda", 0)
    out = []
    for name, rank, hkv in OTHER_CONFIGS:
        gen = torch.Generator(device=dev)
        if name == "prefix_cp4_p4096_e8192":
            ps_ = PREFIX_SHARE
            cp, h_q, h_kv, d, ps = ps_["cp_size"], ps_["h_q"], ps_["h_kv"], ps_["d"], ps_["page_size"]
            lens, prefix = ps_["extend"], ps_["prefix"]
            full = [e + p for e, p in zip(lens, prefix)]
            gen.manual_seed(ps_["seed"] * 100 + rank)
            wp = synth.Workload(name=name, seed=ps_["seed"], causal=True, h_q=h_q, h_kv=h_kv, d=d,
                                page_size=ps, contiguous_kv=False, cp_size=cp)
            meta = cpa.meta_build(cp, rank, lens, seq_lens=full, attn_group=h_q // h_kv, device=dev)
            indptr, indices, n_pages = synth.page_table(wp, full)
            causal = True
        else:
            w = synth.WORKLOADS[name]
            d, ps = w.d, w.page_size
            h_q, h_kv = w.h_q, (hkv or w.h_kv)
            gen.manual_seed(w.seed * 100 + rank)
            causal = w.causal
            if causal:
                lens = synth.sequence_lengths(w)
                meta = cpa.meta_build(w.cp_size, rank, lens, attn_group=h_q // h_kv, device=dev)
                indptr, indices, n_pages = synth.page_table(w, lens)
            else:
                share = w.kv_total // w.ag_degree
                q_start = rank * share
                if w.packed_docs is not None:
                    doc_cu = synth.packed_doc_cu(w)
                    meta = cpa.allgather_packed_meta_build(doc_cu, q_start, share, h_q // h_kv, device=dev)
                else:
                    doc_cu = [0, w.kv_real]
                    meta = cpa.allgather_meta_build(share, max(0, min(share, w.kv_real - q_start)), w.kv_real,
                                                    h_q // h_kv, device=dev)
                n_pages = w.kv_total // ps
                indptr, indices = np.array([0, n_pages], np.int32), np.arange(n_pages, dtype=np.int32)
        q = torch.randn(meta.n_local_rows, h_q, d, generator=gen, device=dev).to(torch.bfloat16)
        kp = torch.randn(n_pages, ps, h_kv, d, generator=gen, device=dev).to(torch.bfloat16)
        vp = torch.randn(n_pages, ps, h_kv, d, generator=gen, device=dev).to(torch.bfloat16)
        if not causal:       # the pad suffix must never be read
            kp.view(-1, h_kv, d)[w.kv_real:] = float("nan")
            vp.view(-1, h_kv, d)[w.kv_real:] = float("nan")
            pairs = sum(max(0, min(doc_cu[b + 1], q_start + share) - max(doc_cu[b], q_start)) *
                        (doc_cu[b + 1] - doc_cu[b]) for b in range(len(doc_cu) - 1))
        else:
            pairs = sum(causal_pairs(qn, kv) for qn, kv in
                        zip(meta.q_prev + meta.q_next, meta.kv_len_prev + meta.kv_len_next))
        ip, ix = torch.from_numpy(indptr).to(dev), torch.from_numpy(indices).to(dev)
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(d)
        flops = 4 * d * h_q * pairs

        def launch():
            cpa.prefill_attn(q, kp, vp, o, meta, scale, ps, ip, ix)
        est = time_launches(torch, launch, 3, 3)
        iters = int(min(400, max(10, 60.0 / max(est, 1e-3))))
        ms = time_launches(torch, launch, max(5, iters // 4), iters)
        if not torch.isfinite(o).all():
            print(f"non-finite attention output on {name} rank {rank}", file=sys.stderr)
            sys.exit(1)
        tf = flops / (ms * 1e-3) / 1e12
        out.append({"workload": name, "rank": rank, "h_q": h_q, "h_kv": h_kv, "page_size": ps,
                    "attn_ms": round(ms, 4), "useful_tflops": round(tf, 1),
                    "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "launches_timed": iters})
        del q, kp, vp, o
    return out


def main():
    args = parse()
    if args.record_traffic:
        import synth
        w = synth.WORKLOADS[args.workload]
        record_traffic(*args.record_traffic, w.name, w.ranks[0] if args.rank is None else args.rank)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the exchange between GPUs is not implemented (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return
    import torch
    import context_prefill_attention_amd as cpa
    import synth

    if args.workload not in synth.WORKLOADS:
        print(f"unknown workload {args.workload}; one of {sorted(synth.WORKLOADS)}", file=sys.stderr)
        sys.exit(2)
    w = synth.WORKLOADS[args.workload]
    if w.causal and (args.kv_heads is not None or args.q_heads is not None):
        print("--kv-heads and --q-heads apply to the AllGather-KV workloads", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    res = run_zigzag(args, w, torch, cpa, synth) if w.causal else run_allgather(args, w, torch, cpa, synth)
    if not args.no_other_configs and args.workload == "long_cp8_s131072_r3":
        res["other_configs"] = other_configs(torch, cpa, synth)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
