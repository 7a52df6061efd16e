"""Run-time job scheduling of cp_prefill_attn (through the C ABI).

With more jobs (work item, KV head) than compute units and items of at least
48 key tiles on average, the first round of workgroups runs jobs 0..n_cu-1 and
every later one draws its job from counters in the metadata blob's header:
one queue per XCD, and an XCD whose queue is empty draws from another.  These
tests size the job count against the device's compute units so that queues
hold one job or none (an XCD must take its job from another's queue), or
several rounds of jobs, and check that every row is written and right, that
outputs are bit-identical from launch to launch, and that the counters are
zero again after every launch."""

import math

import numpy as np
import pytest
import torch

import context_prefill_attention_amd as cpa
import synth
from oracle import attention as oatt
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

CTR_OFFSET, CTR_WORDS = 128, 9    # job counters inside the blob's 256-byte header
ROWS_PER_ITEM = 256


def _n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _counters(meta):
    return meta.d_blob[CTR_OFFSET:CTR_OFFSET + 4 * CTR_WORDS].cpu().view(torch.int32).tolist()


def _jobs_case(n_jobs, h_kv, h_q=32, d=128, kv_len=3072, ps=64, seed=21):
    """AllGather-KV slice whose work list has exactly n_jobs / h_kv items of
    kv_len / 64 key tiles each."""
    group = h_q // h_kv
    q_tile = ROWS_PER_ITEM // group
    assert n_jobs % h_kv == 0
    q_total = n_jobs // h_kv * q_tile
    npages = -(-kv_len // ps)
    qg, kg, vg = synth.normal_bf16(seed, (q_total, h_q, d), (npages * ps, h_kv, d), (npages * ps, h_kv, d))
    meta = cpa.allgather_meta_build(q_total, q_total, kv_len, group, device="cuda")
    assert meta.n_work * h_kv == n_jobs and meta.mean_item_tiles == kv_len // 64
    kp = kg.view(npages, ps, h_kv, d).cuda()
    vp = vg.view(npages, ps, h_kv, d).cuda()
    indptr = torch.tensor([0, npages], dtype=torch.int32, device="cuda")
    indices = torch.arange(npages, dtype=torch.int32, device="cuda")
    return qg, kg, vg, meta, kp, vp, indptr, indices, q_tile


@pytest.mark.parametrize("extra,h_kv,d,ps", [(1, 1, 128, 64), (3, 1, 128, 64), (37, 1, 128, 64), (None, 8, 128, 64),
                                             (37, 1, 64, 16), (None, 8, 64, 32)])
def test_runtime_scheduling_every_job_once(extra, h_kv, d, ps):
    n_cu = _n_cu()
    n_jobs = n_cu + extra if extra is not None else -(-(3 * n_cu + 40) // 8) * 8
    qg, kg, vg, meta, kp, vp, indptr, indices, q_tile = _jobs_case(n_jobs, h_kv, d=d, ps=ps)
    assert n_jobs > n_cu and meta.mean_item_tiles >= 48     # the run-time path is the one taken
    assert _counters(meta) == [0] * CTR_WORDS
    q = qg.cuda()
    scale = 1 / math.sqrt(qg.shape[-1])
    first = None
    for launch in range(3):
        out = torch.full(qg.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        print(f"sched n_jobs={n_jobs} h_kv={h_kv} d={d} ps={ps} launch {launch}", flush=True)
        cpa.prefill_attn(q, kp, vp, out, meta, scale, ps, indptr, indices)
        torch.cuda.synchronize()
        assert _counters(meta) == [0] * CTR_WORDS, f"counters left set after launch {launch}"
        assert torch.isfinite(out).all(), "a job was not run (rows still hold the NaN fill)"
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), "launches differ"
    # parity on rows of the first items, the last items (drawn at run time) and spread between
    n_items = n_jobs // h_kv
    rng = np.random.default_rng(n_jobs)
    items = sorted({0, 1, n_items - 2, n_items - 1} | set(rng.integers(0, n_items, 12).tolist()))
    rows = sorted({it * q_tile + int(rng.integers(0, q_tile)) for it in items})
    ref = oatt.allgather_kv(qg, kg, vg, qg.shape[0], 3072, scale, rows=rows)
    err = gc.assert_close(first[rows], ref, f"sched n_jobs={n_jobs}")
    print("sched", n_jobs, h_kv, "err", err, flush=True)


def test_static_path_leaves_counters_alone():
    """Items under 48 key tiles: every workgroup runs its own job, the
    counters are never touched."""
    n_cu = _n_cu()
    qg, kg, vg, meta, kp, vp, indptr, indices, q_tile = _jobs_case(n_cu + 40, 1, kv_len=1024)
    assert meta.mean_item_tiles == 16
    out = torch.full(qg.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(qg.shape[-1])
    cpa.prefill_attn(qg.cuda(), kp, vp, out, meta, scale, 64, indptr, indices)
    torch.cuda.synchronize()
    assert _counters(meta) == [0] * CTR_WORDS
    assert torch.isfinite(out).all()
    rows = [0, 5, qg.shape[0] // 2, qg.shape[0] - 1]
    gc.assert_close(out[rows], oatt.allgather_kv(qg, kg, vg, qg.shape[0], 1024, scale, rows=rows), "static")


def test_runtime_scheduling_in_a_graph():
    """The attention launch captured in a HIP graph: each replay finds the
    counters at zero (the previous replay's last ticket taker cleared them)
    and gives the eager result bit for bit."""
    n_cu = _n_cu()
    qg, kg, vg, meta, kp, vp, indptr, indices, q_tile = _jobs_case(n_cu + 37, 1)
    q = qg.cuda()
    scale = 1 / math.sqrt(qg.shape[-1])
    out = torch.empty(qg.shape, dtype=torch.bfloat16, device="cuda")

    def step():
        cpa.prefill_attn(q, kp, vp, out, meta, scale, 64, indptr, indices)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"sched graph replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert _counters(meta) == [0] * CTR_WORDS, f"replay {rep}: counters left set"
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        step()   # eager launch between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"eager after replay {rep}"


@pytest.mark.parametrize("seed", range(16))
def test_runtime_scheduling_random_shapes(seed):
    """Seeded AllGather-KV shapes with 1-4 rounds of jobs beyond the CU count,
    every head grouping, D 64/128, pages of 16/64 and a ragged last item: two
    launches of each entry point give the same bits, every row is written,
    the blob counters are zero after each, and sampled rows match the oracle."""
    rng = np.random.default_rng(9000 + seed)
    n_cu = _n_cu()
    h_kv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    h_q, d, ps = h_kv * group, int(rng.choice([64, 128])), int(rng.choice([16, 64]))
    q_tile = ROWS_PER_ITEM // group
    n_items = int(rng.integers(n_cu // h_kv + 1, 4 * n_cu // h_kv + 2))
    q_total = n_items * q_tile - int(rng.integers(0, q_tile))
    kv_len = int(rng.integers(3072, 8193))
    npages = -(-kv_len // ps)
    qg, kg, vg = synth.normal_bf16(9100 + seed, (q_total, h_q, d), (npages * ps, h_kv, d), (npages * ps, h_kv, d))
    meta = cpa.allgather_meta_build(q_total, q_total, kv_len, group, device="cuda")
    assert meta.n_work * h_kv > n_cu and meta.mean_item_tiles >= 48
    print(f"sched random {seed}: H {h_q}/{h_kv} d {d} ps {ps} rows {q_total} keys {kv_len} "
          f"jobs {meta.n_work * h_kv}", flush=True)
    kp, vp = kg.view(npages, ps, h_kv, d).cuda(), vg.view(npages, ps, h_kv, d).cuda()
    ip = torch.tensor([0, npages], dtype=torch.int32, device="cuda")
    ix = torch.arange(npages, dtype=torch.int32, device="cuda")
    q, scale = qg.cuda(), 1 / math.sqrt(d)
    outs = []
    for _launch in range(2):
        for noalloc in (False, True):
            out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
            cpa.prefill_attn(q, kp, vp, out, meta, scale, ps, ip, ix, noalloc=noalloc)
            torch.cuda.synchronize()
            assert torch.isfinite(out).all(), "a job was not run"
            assert _counters(meta) == [0] * CTR_WORDS
            outs.append(out)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    rows = sorted({0, q_total - 1} | set(rng.integers(0, q_total, 4).tolist()))
    gc.assert_close(outs[0][rows], oatt.allgather_kv(qg, kg, vg, q_total, kv_len, scale, rows=rows),
                    f"sched random {seed}")
