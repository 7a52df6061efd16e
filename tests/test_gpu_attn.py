"""GPU parity of cp_prefill_attn against the fp64 oracle (through the C ABI)."""

import math
import random

import numpy as np
import pytest
import torch

import context_prefill_attention_amd as cpa
import synth
from oracle import attention as oatt
from oracle import zigzag_meta
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _tiny_variants():
    rng = random.Random(5)
    out = []
    for cp in (2, 3, 4, 8):
        for _ in range(3):
            bs = rng.randint(1, 3)
            lens = [rng.randint(2 * cp, 2 * cp * 40 + 13) for _ in range(bs)]   # uneven, ragged
            h_kv = rng.choice([1, 2, 4])
            g = rng.choice([1, 2, 3, 8])
            out.append((cp, lens, h_kv * g, h_kv, rng.choice([64, 128]), rng.choice([1, 16, 64])))
    return out


@pytest.mark.parametrize("cp,lens,h_q,h_kv,d,ps", _tiny_variants())
def test_tiny_all_ranks_all_rows(cp, lens, h_q, h_kv, d, ps):
    base = synth.Workload(name="tiny", seed=11, causal=True, h_q=h_q, h_kv=h_kv, d=d, page_size=ps,
                          contiguous_kv=False, cp_size=cp, ranks=tuple(range(cp)), bs=len(lens))
    print(f"tiny cp={cp} lens={lens} H={h_q}/{h_kv} D={d} ps={ps}", flush=True)
    for r in range(cp):
        c = gc.zigzag_case(base, r, lens=lens)
        got = gc.run_attn(c)
        ref = oatt.zigzag_rank(c.q_local.cpu(), c.k_seqs, c.v_seqs, c.meta_o, c.scale)
        gc.assert_close(got, ref, f"rank {r}")


def test_config1_tiny_cp2_s256_both_ranks():
    w = W["tiny_cp2_s256"]
    for r in w.ranks:
        c = gc.zigzag_case(w, r)
        got = gc.run_attn(c)
        ref = oatt.zigzag_rank(c.q_local.cpu(), c.k_seqs, c.v_seqs, c.meta_o, c.scale)
        print("cfg1 rank", r, "max abs/rel err", gc.assert_close(got, ref, f"cfg1 rank {r}"), flush=True)


def test_config2_gqa_cp2_s8192_each_rank():
    w = W["gqa_cp2_s8192"]
    for r in w.ranks:
        c = gc.zigzag_case(w, r)
        got = gc.run_attn(c)
        rows = gc.sample_rows(c.meta_o, c.meta.q_tile, 96, seed=r)
        ref = gc.oracle_rows(c, rows)
        print("cfg2 rank", r, len(rows), "rows, err", gc.assert_close(got[rows], ref, f"cfg2 rank {r}"), flush=True)


def test_config3_varlen_cp4_bs8_all_ranks():
    w = W["varlen_cp4_bs8"]
    for r in w.ranks:
        c = gc.zigzag_case(w, r)
        got = gc.run_attn(c)
        rows = gc.sample_rows(c.meta_o, c.meta.q_tile, 48, seed=10 + r)
        ref = gc.oracle_rows(c, rows)
        print("cfg3 rank", r, len(rows), "rows, err", gc.assert_close(got[rows], ref, f"cfg3 rank {r}"), flush=True)


def test_config4_long_cp8_s131072_rank3_sampled_and_properties():
    w = W["long_cp8_s131072_r3"]
    c = gc.zigzag_case(w, 3, q_global=False)
    got = gc.run_attn(c)
    # properties at full size: finite, and every output is a convex combination of V rows
    assert torch.isfinite(got).all()
    vmax = max(float(c.v_seqs[0].abs().max()), 1e-6)
    assert float(got.abs().max()) <= vmax * (1 + 2 ** -7)
    # Every row (all 64 heads) of four whole work items: the first and last
    # item of each half.  The last next-half item (local rows 16352-16383)
    # is the 1664-tile diagonal item the longest-first list sends out first;
    # the last prev-half item holds that half's diagonal.  Plus 64 random
    # rows, 32 in each half.
    q_tile = c.meta.q_tile
    n_prev = c.meta.total_q_prev_tokens
    n_loc = c.meta.n_local_rows
    items = [0, n_prev - q_tile, n_prev, n_loc - q_tile]
    assert q_tile == 32 and items == [0, 8160, 8192, 16352]
    rows = set()
    for r0 in items:
        rows.update(range(r0, r0 + q_tile))
    rng = np.random.default_rng(4)
    rows.update(int(x) for x in rng.integers(0, n_prev, 32))
    rows.update(int(x) for x in rng.integers(n_prev, n_loc, 32))
    rows = sorted(rows)
    assert len(rows) >= 4 * 32 + 60
    ref = gc.oracle_rows(c, rows)
    print("cfg4", len(rows), "rows, err", gc.assert_close(got[rows], ref, "cfg4"), flush=True)
    # determinism: a second launch gives identical bits
    got2 = gc.run_attn(c)
    assert torch.equal(got.view(torch.int16), got2.view(torch.int16))


def _allgather_case(h_kv, q_real=None, q_total=8192, rows_from=8192, kv_total=32768, kv_real=30000,
                    ps=64, seed=5):
    w = W["allgather_kv_s32768"]
    d, h_q = w.d, w.h_q
    qg, kg, vg = synth.normal_bf16(seed, (kv_total, h_q, d), (kv_total, h_kv, d), (kv_total, h_kv, d))
    q = qg[rows_from:rows_from + q_total].contiguous()
    kg[kv_real:] = float("nan")      # the pad suffix must never be read
    vg[kv_real:] = float("nan")
    q_real = q_total if q_real is None else q_real
    meta = cpa.allgather_meta_build(q_total, q_real, kv_real, h_q // h_kv, device="cuda")
    npages = kv_total // ps
    kp = kg.view(npages, ps, h_kv, d).cuda()
    vp = vg.view(npages, ps, h_kv, d).cuda()
    indptr = torch.tensor([0, npages], dtype=torch.int32, device="cuda")
    indices = torch.arange(npages, dtype=torch.int32, device="cuda")
    out = torch.full((q_total, h_q, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(d)
    cpa.prefill_attn(q.cuda(), kp, vp, out, meta, scale, ps, indptr, indices)
    torch.cuda.synchronize()
    return q, kg, vg, out, scale, q_real


@pytest.mark.parametrize("h_kv", [8, 1])
def test_config5_allgather_kv(h_kv):
    q, kg, vg, out, scale, q_real = _allgather_case(h_kv)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(h_kv)
    rows = sorted(set([0, 1, 63, 64, 127, 4095, 8191]) | set(rng.integers(0, 8192, 40).tolist()))
    ref = oatt.allgather_kv(q, kg, vg, q_real, 30000, scale, rows=rows)
    print("cfg5 H_kv", h_kv, "err", gc.assert_close(out[rows], ref, f"cfg5 hkv={h_kv}"), flush=True)


@pytest.mark.parametrize("h_kv,q_real,q_total,kv_real", [(8, 700, 1000, 1234), (1, 1, 40, 1), (2, 0, 64, 77)])
def test_allgather_pad_rows_and_ragged(h_kv, q_real, q_total, kv_real):
    q, kg, vg, out, scale, q_real = _allgather_case(h_kv, q_real=q_real, q_total=q_total, rows_from=0,
                                                     kv_total=2048, kv_real=kv_real, ps=16, seed=7)
    ref = oatt.allgather_kv(q, kg, vg, q_real, kv_real, scale)
    gc.assert_close(out, ref, "allgather ragged")
    assert torch.all(out[q_real:] == 0)


def _prefix_extend_case(cp, lens, prefix, h_q, h_kv, d, ps, seed, sample=None):
    """Cached prefix ahead of the extend part: kv_len grows by the prefix and
    the causal alignment stays bottom-right.  The pool holds prefix and
    extend keys of every sequence (filled by plain indexing); ``sample`` rows
    per rank are compared (None: every row)."""
    full = [p + e for p, e in zip(prefix, lens)]
    bs = len(lens)
    qg, kg, vg = synth.normal_bf16(seed, (sum(full), h_q, d), (sum(full), h_kv, d), (sum(full), h_kv, d))
    starts = np.concatenate([[0], np.cumsum(full)])
    k_seqs = [kg[starts[b]:starts[b + 1]] for b in range(bs)]
    v_seqs = [vg[starts[b]:starts[b + 1]] for b in range(bs)]
    q_ext = torch.cat([qg[starts[b] + prefix[b]:starts[b + 1]] for b in range(bs)])
    w = synth.Workload(name="pfx", seed=seed, causal=True, h_q=h_q, h_kv=h_kv, d=d, page_size=ps,
                       contiguous_kv=False, cp_size=cp)
    indptr, indices, npages = synth.page_table(w, full)
    rows = gc.pool_rows(full, prefix, indptr, indices, ps)
    kp = torch.zeros(npages * ps, h_kv, d, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    for b in range(bs):
        kp[torch.from_numpy(rows[b])] = k_seqs[b]
        vp[torch.from_numpy(rows[b])] = v_seqs[b]
    kp, vp = kp.view(npages, ps, h_kv, d).cuda(), vp.view(npages, ps, h_kv, d).cuda()
    from oracle import layout
    for r in range(cp):
        mo = zigzag_meta.build(cp, r, sum(lens), seq_lens=full, extend_lens=lens)
        q_loc = torch.from_numpy(layout.shard(q_ext.view(torch.int16).numpy(), mo)).view(torch.bfloat16)
        meta = cpa.meta_build(cp, r, lens, seq_lens=full, attn_group=h_q // h_kv, device="cuda")
        out = torch.full(q_loc.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        cpa.prefill_attn(q_loc.cuda(), kp, vp, out, meta, 1 / math.sqrt(d), ps, torch.from_numpy(indptr).cuda(),
                         torch.from_numpy(indices).cuda())
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), f"prefix rank {r}: rows left unwritten"   # every job ran
        if sample is None:
            ref = oatt.zigzag_rank(q_loc, k_seqs, v_seqs, mo, 1 / math.sqrt(d))
            gc.assert_close(out, ref, f"prefix rank {r}")
        else:
            loc = gc.sample_rows(mo, meta.q_tile, sample, seed + r)
            ref = oatt.zigzag_rank_rows(q_loc, loc, k_seqs, v_seqs, mo, 1 / math.sqrt(d))
            print("prefix rank", r, "err", gc.assert_close(out[loc], ref, f"prefix rank {r}"), flush=True)


def test_prefix_extend_kv_includes_cached_prefix():
    _prefix_extend_case(2, [96, 40], [64, 0], 8, 2, 128, 16, 31)


def test_prefix_extend_p4096_e8192_cp4_sampled():
    """Prefix-cached extend at size: a 4096-token cached prefix ahead of an
    8192-token extend, next to a sequence without prefix (6144 tokens), cp = 4,
    GQA 32/4, pages of 64 with permuted ids; sampled rows of every rank."""
    _prefix_extend_case(4, [8192, 6144], [4096, 0], 32, 4, 128, 64, 41, sample=24)


def test_mha_and_mqa_group_shapes():
    for h_q, h_kv in ((4, 4), (16, 1), (64, 8)):
        base = synth.Workload(name="grp", seed=13, causal=True, h_q=h_q, h_kv=h_kv, d=128, page_size=16,
                              contiguous_kv=False, cp_size=2)
        c = gc.zigzag_case(base, 1, lens=[520])
        got = gc.run_attn(c)
        ref = oatt.zigzag_rank(c.q_local.cpu(), c.k_seqs, c.v_seqs, c.meta_o, c.scale)
        gc.assert_close(got, ref, f"H {h_q}/{h_kv}")


def _packed_run(doc_cu, q_start, q_total, h_q, h_kv, d, ps, kv_total, seed, permute):
    """Packed AllGather-KV share: global K/V [kv_total] (pad suffix NaN) as a
    pool of pages, identity or permuted page ids; local Q = global rows
    [q_start, q_start + q_total)."""
    qg, kg, vg = synth.normal_bf16(seed, (kv_total, h_q, d), (kv_total, h_kv, d), (kv_total, h_kv, d))
    real = doc_cu[-1]
    kg[real:] = float("nan")
    vg[real:] = float("nan")
    q = qg[q_start:q_start + q_total].contiguous()
    meta = cpa.allgather_packed_meta_build(doc_cu, q_start, q_total, h_q // h_kv, device="cuda")
    npages = kv_total // ps
    ids = np.random.default_rng(seed + 1000).permutation(npages) if permute else np.arange(npages)
    kp = torch.empty(npages, ps, h_kv, d, dtype=torch.bfloat16)
    vp = torch.empty_like(kp)
    kp[torch.from_numpy(ids)] = kg.view(npages, ps, h_kv, d)   # logical page i lives at pool page ids[i]
    vp[torch.from_numpy(ids)] = vg.view(npages, ps, h_kv, d)
    indptr = torch.tensor([0, npages], dtype=torch.int32, device="cuda")
    indices = torch.from_numpy(ids.astype(np.int32)).cuda()
    out = torch.full((q_total, h_q, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    scale = 1 / math.sqrt(d)
    cpa.prefill_attn(q.cuda(), kp.cuda(), vp.cuda(), out, meta, scale, ps, indptr, indices)
    torch.cuda.synchronize()
    return q, kg, vg, out, scale


def _packed_tiny_variants():
    cu = [0, 37, 137, 142, 442, 506]      # uneven documents, one of 5 tokens; pad 506..575
    out = []
    for d in (64, 128):
        for ps, permute in ((16, False), (64, False), (64, True), (16, True)):
            out.append((cu, 576, 4, 8, 2, d, ps, permute))
    out.append(([0, 1, 2, 70, 200], 256, 2, 4, 1, 64, 64, True))     # one-token documents, MQA
    out.append(([0, 500], 512, 8, 4, 4, 128, 16, False))               # one document, MHA
    # documents starting on page boundaries (a tile's pages are whole pages of
    # one document's row range), and one aligned only to half a page
    out.append(([0, 64, 96, 352, 480], 576, 4, 8, 2, 128, 32, True))
    out.append(([0, 48, 64, 208, 400, 464], 576, 4, 8, 2, 128, 16, True))
    out.append(([0, 8, 136, 200, 504], 576, 4, 8, 1, 64, 8, True))
    out.append(([0, 48, 208, 512], 576, 4, 8, 2, 128, 32, True))
    return out


@pytest.mark.parametrize("cu,kv_total,a,h_q,h_kv,d,ps,permute", _packed_tiny_variants())
def test_allgather_packed_tiny_all_ranks_all_rows(cu, kv_total, a, h_q, h_kv, d, ps, permute):
    """Every rank's slice of a packed sequence, every row: documents starting
    at unaligned keys (tiles straddle page boundaries) or on page boundaries
    of 8, 16 or 32 keys; pad rows are zero."""
    share = kv_total // a
    for r in range(a):
        q, kg, vg, out, scale = _packed_run(cu, r * share, share, h_q, h_kv, d, ps, kv_total, 31 + r, permute)
        ref = oatt.allgather_kv_packed(q, kg, vg, cu, r * share, scale)
        gc.assert_close(out, ref, f"packed rank {r} d={d} ps={ps} permute={permute}")
        pad0 = max(0, cu[-1] - r * share)
        assert torch.all(out[pad0:] == 0)


@pytest.mark.parametrize("rank,h_q,h_kv", [(1, 32, 8), (3, 32, 8), (1, 32, 1), (1, 16, 4), (3, 16, 4)])
def test_allgather_packed_s32768_sampled(rank, h_q, h_kv):
    """The packed AllGather-KV workload at full size (7 documents in 30000 real
    rows of 32768, A = 4): ranks 1 (four documents) and 3 (two documents and
    the pad suffix), GQA, MQA and the Ulysses U = 2 head share (16/4).  Rows
    around every document boundary, the slice ends and random rows."""
    w = W["allgather_packed_s32768"]
    cu = synth.packed_doc_cu(w)
    share = w.kv_total // w.ag_degree
    q0 = rank * share
    q, kg, vg, out, scale = _packed_run(cu, q0, share, h_q, h_kv, w.d, w.page_size, w.kv_total, w.seed, False)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(rank * 100 + h_kv)
    rows = {0, 1, share - 1} | set(rng.integers(0, share, 24).tolist())
    for c in cu:
        for dr in (-1, 0, 1):
            if 0 <= c - q0 + dr < share:
                rows.add(c - q0 + dr)
    rows = sorted(rows)
    ref = oatt.allgather_kv_packed(q, kg, vg, cu, q0, scale, rows=rows)
    print("packed rank", rank, "heads", h_q, h_kv, "err", gc.assert_close(out[rows], ref, "packed s32768"), flush=True)
    if q0 + share > cu[-1]:
        assert torch.all(out[cu[-1] - q0:] == 0)


@pytest.mark.parametrize("ps,d", [(2, 128), (4, 64), (8, 128), (16, 64), (32, 128), (32, 64),
                                  (128, 128), (256, 64)])
def test_page_sizes(ps, d):
    """Page sizes below, at and above the 64-key tile, at both head sizes:
    per-lane page lookups (ps < 16), whole pages per tile (ps 16 and 32),
    and one page per tile or several tiles per page (ps >= 64); pages
    permuted; every rank of a ragged two-sequence batch, every row."""
    w = synth.Workload(name=f"ps{ps}", seed=50 + ps + d, causal=True, h_q=8, h_kv=2, d=d,
                       page_size=ps, contiguous_kv=False, cp_size=3)
    lens = [1237, 419]
    for r in range(3):
        c = gc.zigzag_case(w, r, lens=lens)
        out = gc.run_attn(c)
        ref = oatt.zigzag_rank(c.q_local.cpu(), c.k_seqs, c.v_seqs, c.meta_o, c.scale)
        gc.assert_close(out, ref, f"ps={ps} d={d} rank {r}")


def _sweep_params(seed):
    """Random small shapes: cp, ragged lengths, optional cached prefixes, head
    groups, head size and page size (every page mode), drawn from the seed."""
    rng = np.random.default_rng(1000 + seed)
    cp = int(rng.choice([2, 3, 4, 5, 8]))
    bs = int(rng.integers(1, 4))
    lens = [int(rng.integers(2 * cp, 2 * cp + 300)) for _ in range(bs)]
    prefix = [int(rng.integers(0, 200)) if rng.random() < 0.4 else 0 for _ in range(bs)]
    h_kv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([64, 128]))
    ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    return cp, lens, prefix, h_kv * group, h_kv, d, ps


@pytest.mark.parametrize("seed", range(48))
def test_random_zigzag_sweep_all_ranks_all_rows(seed):
    """Seeded random shapes through the whole causal path, every rank and row."""
    cp, lens, prefix, h_q, h_kv, d, ps = _sweep_params(seed)
    print("sweep", seed, "cp", cp, "lens", lens, "prefix", prefix, "heads", h_q, h_kv, "d", d, "ps", ps,
          flush=True)
    _prefix_extend_case(cp, lens, prefix, h_q, h_kv, d, ps, 500 + seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_packed_allgather_sweep(seed):
    """Seeded random packed AllGather-KV slices: document lengths (some
    page-aligned, some not), pad suffix, degree, heads, head and page size;
    every rank, every row."""
    rng = np.random.default_rng(2000 + seed)
    ps = int(rng.choice([4, 16, 32, 64]))
    a = int(rng.choice([2, 3, 4]))
    m = int(np.lcm(a, ps))     # the slices split evenly and the pool holds whole pages
    kv_total = m * int(rng.integers(max(2, 48 // m), max(3, 640 // m)))
    align = ps if rng.random() < 0.5 else 1
    cu = [0]
    while True:
        n = align * int(rng.integers(1, max(2, 200 // align)))
        if cu[-1] + n >= kv_total:
            break
        cu.append(cu[-1] + n)
    if rng.random() < 0.5 or len(cu) == 1:
        end = kv_total - int(rng.integers(0, min(40, kv_total // 4)))   # a pad suffix
        if end > cu[-1]:
            cu.append(end)
    h_kv = int(rng.choice([1, 2]))
    h_q = h_kv * int(rng.choice([1, 4, 8]))
    d = int(rng.choice([64, 128]))
    share = kv_total // a
    print("packed sweep", seed, "cu", cu, "kv_total", kv_total, "a", a, "heads", h_q, h_kv, "d", d, "ps", ps,
          flush=True)
    for r in range(a):
        q, kg, vg, out, scale = _packed_run(cu, r * share, share, h_q, h_kv, d, ps, kv_total, 3000 + seed,
                                            permute=True)
        ref = oatt.allgather_kv_packed(q, kg, vg, cu, r * share, scale)
        gc.assert_close(out, ref, f"packed sweep {seed} rank {r}")
        pad0 = max(0, cu[-1] - r * share)
        assert torch.all(out[pad0:] == 0)


@pytest.mark.parametrize("seed", range(24))
def test_random_midsize_sweep_sampled(seed):
    """Seeded mid-size causal shares (2k-12k tokens per sequence, so the
    unmasked key loop runs many unrolled iterations) in every page mode;
    sampled rows of every rank, including each work item's first and last."""
    rng = np.random.default_rng(4000 + seed)
    cp = int(rng.choice([2, 4, 8]))
    bs = int(rng.integers(1, 3))
    lens = [int(rng.integers(2048, 12289)) for _ in range(bs)]
    prefix = [int(rng.integers(0, 3000)) if rng.random() < 0.3 else 0 for _ in range(bs)]
    h_kv = int(rng.choice([1, 2, 4]))
    h_q = h_kv * int(rng.choice([1, 4, 8]))
    d = int(rng.choice([64, 128]))
    ps = int(rng.choice([4, 16, 32, 64, 256]))
    print("midsize", seed, "cp", cp, "lens", lens, "prefix", prefix, "heads", h_q, h_kv, "d", d, "ps", ps,
          flush=True)
    _prefix_extend_case(cp, lens, prefix, h_q, h_kv, d, ps, 6000 + seed, sample=6)


def test_meta_buffers_reused_without_allocation_and_stream_ordered():
    """Metadata uploaded through one reusable MetaBuffers, alternating ranks
    with no synchronisation between the launches: every launch reads the
    metadata built for it (stream order), the outputs are bit-identical to
    those with freshly allocated metadata, and no torch allocation happens
    once the buffers exist."""
    w = W["tiny_cp2_s256"]
    cases = [gc.zigzag_case(w, r) for r in w.ranks]
    ref = [gc.run_attn(c) for c in cases]
    mb = cpa.MetaBuffers("cuda")
    outs = [torch.empty_like(c.q_local) for c in cases]
    lens = cases[0].lens
    group = w.h_q // w.h_kv

    def one_round():
        for r, c in enumerate(cases):
            m = cpa.meta_build(w.cp_size, c.rank, lens, attn_group=group, buffers=mb)
            outs[r].fill_(float("nan"))
            cpa.prefill_attn(c.q_local, c.k_pool, c.v_pool, outs[r], m, c.scale, c.extra["page_size"],
                             c.indptr, c.indices)
    one_round()
    torch.cuda.synchronize()
    allocs = torch.cuda.memory_stats()["allocation.all.allocated"]
    for _ in range(5):
        one_round()
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == allocs
    for r in range(len(cases)):
        assert torch.equal(outs[r].view(torch.int16), ref[r].view(torch.int16)), f"rank {r}"


@pytest.mark.parametrize("gap,what", [(40.0, "~650 above the first block"),
                                      (6.125, "~100 above the first block")])
def test_late_keys_far_above_the_first_block(gap, what):
    """Scores of later keys far above every score of the item's first key
    block, which sets the softmax reference.  With q = 1 and k = gap in every
    dimension the score is 128 * gap / sqrt(128) above the first block's
    (k = 0): about 650 in the exp2 domain for gap 40 (the probabilities
    against the old reference would overflow fp32, so the lazy reference
    must be raised, and O and l rescaled, mid-item) and about 100 for gap
    6.125.  Both must match the oracle."""
    cp, lens, h_q, h_kv, d, ps = 2, [512], 4, 1, 128, 16
    total = sum(lens)
    qg, kg, vg = synth.normal_bf16(77, (total, h_q, d), (total, h_kv, d), (total, h_kv, d))
    kg[:64] = 0.0                    # the first key tile scores 0 against any query
    qg[:] = 1.0
    kg[100:110] = gap                # a few keys far above it, early in the sequence
    kg[400:404] = gap                # and late
    base = synth.Workload(name="gap", seed=77, causal=True, h_q=h_q, h_kv=h_kv, d=d, page_size=ps,
                          contiguous_kv=True, cp_size=cp, ranks=(0, 1), bs=1)
    for r in range(cp):
        c = gc.zigzag_case(base, r, lens=lens)
        mo = c.meta_o
        from oracle import layout
        c.q_local = torch.from_numpy(layout.shard(gc.bits(qg), mo)).view(torch.bfloat16).cuda()
        c.k_seqs, c.v_seqs = [kg], [vg]
        c.k_pool = kg.view(total // ps, ps, h_kv, d).cuda()
        c.v_pool = vg.view(total // ps, ps, h_kv, d).cuda()
        got = gc.run_attn(c)
        ref = oatt.zigzag_rank(c.q_local.cpu(), c.k_seqs, c.v_seqs, mo, c.scale)
        print(what, "rank", r, "err", gc.assert_close(got, ref, f"gap {gap} rank {r}"), flush=True)


def test_concurrent_streams_independent():
    """The library keeps no device state between calls: the whole step of two
    different shares (metadata, scatter, paired rerange, attention), issued on
    two streams at once, gives the same bits as one share at a time."""
    w = W["gqa_cp2_s8192"]
    cases = [gc.zigzag_case(w, r, q_global=False) for r in w.ranks]
    ref = [gc.run_attn(c) for c in cases]
    n_g = w.cp_size * cases[0].meta.max_rank_len
    total = sum(cases[0].lens)
    gens = [torch.Generator(device="cuda").manual_seed(90 + i) for i in range(2)]
    k_gath = [torch.randn(n_g, w.h_kv, w.d, generator=g, device="cuda").to(torch.bfloat16) for g in gens]
    v_gath = [torch.randn(n_g, w.h_kv, w.d, generator=g, device="cuda").to(torch.bfloat16) for g in gens]
    ko_ref = [torch.empty(total, w.h_kv, w.d, dtype=torch.bfloat16, device="cuda") for _ in cases]
    vo_ref = [torch.empty_like(t) for t in ko_ref]
    for c, kg, vg, ko, vo in zip(cases, k_gath, v_gath, ko_ref, vo_ref):
        cpa.zigzag_rerange_kv(c.meta, kg, ko, vg, vo, cpa.GATHERED_TO_ORIG)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [torch.full_like(c.q_local, float("nan")) for c in cases]
    ko = [torch.full_like(t, float("nan")) for t in ko_ref]
    vo = [torch.full_like(t, float("nan")) for t in vo_ref]
    for _ in range(3):
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                m = cpa.meta_build(w.cp_size, c.rank, c.lens, attn_group=w.h_q // w.h_kv, device="cuda")
                cpa.zigzag_rerange_kv(m, k_gath[i], ko[i], v_gath[i], vo[i], cpa.GATHERED_TO_ORIG)
                cpa.prefill_attn(c.q_local, c.k_pool, c.v_pool, outs[i], m, c.scale, c.extra["page_size"],
                                 c.indptr, c.indices)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16)), f"rank {c.rank}"
        assert torch.equal(ko[i].view(torch.int16), ko_ref[i].view(torch.int16))
        assert torch.equal(vo[i].view(torch.int16), vo_ref[i].view(torch.int16))
