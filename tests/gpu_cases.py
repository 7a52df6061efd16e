"""Inputs and oracle expectations for the GPU parity tests.

Inputs come from ``synth`` (seeded); expected values come only from
``oracle``.  The HIP path is called only through the package binding (C ABI).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import context_prefill_attention_amd as cpa
import synth
from oracle import attention as oatt
from oracle import layout, zigzag_meta

ATOL = 1e-2
RTOL = 1e-2
BF16_NAN_BITS = np.int16(0x7FC0)


def assert_close(got, ref, what=""):
    """|got - ref| <= 1e-2 + 1e-2*|ref| elementwise (bf16 output vs fp64 oracle)."""
    g = got.detach().float().cpu().numpy().astype(np.float64) if hasattr(got, "detach") else np.asarray(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; max abs err "
                             f"{err.max():.3e}; first at {idx.tolist()}")
    return float(err.max()), float((err / np.maximum(np.abs(r), 1e-30)).max())


def bits(t: torch.Tensor) -> np.ndarray:
    """int16 bit pattern of a bf16 tensor (CPU numpy)."""
    return t.detach().cpu().view(torch.int16).numpy()


def pool_rows(kv_lens, prefix, indptr, indices, page_size):
    """Flat pool row (page*page_size + slot) of every sequence position, per sequence."""
    out = []
    for b, n in enumerate(kv_lens):
        pos = np.arange(n)
        out.append(indices[indptr[b] + pos // page_size].astype(np.int64) * page_size + pos % page_size)
    return out


@dataclass
class ZigzagCase:
    w: synth.Workload
    rank: int
    lens: List[int]
    meta_o: zigzag_meta.ZigzagMeta
    meta: cpa.Meta
    q_local: torch.Tensor          # device
    k_seqs: List[torch.Tensor]     # CPU bf16, per sequence
    v_seqs: List[torch.Tensor]
    k_pool: torch.Tensor           # device
    v_pool: torch.Tensor
    indptr: torch.Tensor
    indices: torch.Tensor
    num_pages: int
    scale: float
    extra: dict = field(default_factory=dict)


def zigzag_case(w: synth.Workload, rank: int, device="cuda", q_global: bool = True,
                lens: Optional[List[int]] = None, h_q=None, h_kv=None, d=None,
                page_size=None, seed=None) -> ZigzagCase:
    """One rank's share: local Q, per-sequence K/V and a paged pool filled by
    plain torch indexing (independent of the scatter kernel)."""
    h_q = h_q or w.h_q
    h_kv = h_kv or w.h_kv
    d = d or w.d
    ps = page_size or w.page_size
    seed = w.seed if seed is None else seed
    lens = lens or synth.sequence_lengths(w)
    total = sum(lens)
    mo = zigzag_meta.build(w.cp_size, rank, total, extend_lens=lens)
    if q_global:
        qg, kg, vg = synth.normal_bf16(seed, (total, h_q, d), (total, h_kv, d), (total, h_kv, d))
        q_loc = torch.from_numpy(layout.shard(qg.view(torch.int16).numpy(), mo)).view(torch.bfloat16)
    else:
        n_loc = mo.per_rank_actual_token[rank]
        q_loc, kg, vg = synth.normal_bf16(seed, (n_loc, h_q, d), (total, h_kv, d), (total, h_kv, d))
    starts = np.concatenate([[0], np.cumsum(lens)])
    k_seqs = [kg[starts[b]:starts[b + 1]] for b in range(len(lens))]
    v_seqs = [vg[starts[b]:starts[b + 1]] for b in range(len(lens))]
    wp = synth.Workload(**{**w.__dict__, "page_size": ps})
    indptr, indices, n_pages = synth.page_table(wp, lens)
    rows = pool_rows(lens, [0] * len(lens), indptr, indices, ps)
    k_pool = torch.zeros(n_pages * ps, h_kv, d, dtype=torch.bfloat16)
    v_pool = torch.zeros(n_pages * ps, h_kv, d, dtype=torch.bfloat16)
    for b in range(len(lens)):
        k_pool[torch.from_numpy(rows[b])] = k_seqs[b]
        v_pool[torch.from_numpy(rows[b])] = v_seqs[b]
    meta = cpa.meta_build(w.cp_size, rank, lens, attn_group=h_q // h_kv, device=device)
    return ZigzagCase(
        w=w, rank=rank, lens=lens, meta_o=mo, meta=meta, q_local=q_loc.to(device),
        k_seqs=k_seqs, v_seqs=v_seqs,
        k_pool=k_pool.view(n_pages, ps, h_kv, d).to(device),
        v_pool=v_pool.view(n_pages, ps, h_kv, d).to(device),
        indptr=torch.from_numpy(indptr).to(device), indices=torch.from_numpy(indices).to(device),
        num_pages=n_pages, scale=1.0 / math.sqrt(d), extra={"page_size": ps})


def run_attn(c: ZigzagCase) -> torch.Tensor:
    out = torch.full_like(c.q_local, float("nan"))
    cpa.prefill_attn(c.q_local, c.k_pool, c.v_pool, out, c.meta, c.scale, c.extra["page_size"],
                     c.indptr, c.indices)
    torch.cuda.synchronize()
    return out


def sample_rows(mo: zigzag_meta.ZigzagMeta, q_tile: int, n_random: int, seed: int) -> List[int]:
    """Local rows worth checking: each segment's first/last rows, the rows at
    work-item edges (multiples of q_tile), and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for _h, _b, r0, q_len, _kv in zigzag_meta.segments(mo):
        for p in (0, 1, q_len - 2, q_len - 1, q_len // 2):
            if 0 <= p < q_len:
                rows.add(r0 + p)
        for p in range(0, q_len, q_tile):
            rows.update({r0 + p, r0 + min(q_len - 1, p + q_tile - 1)})
    rows = sorted(rows)
    if len(rows) > 3 * n_random:
        rows = sorted(rng.choice(rows, 3 * n_random, replace=False).tolist())
    extra = rng.integers(0, mo.per_rank_actual_token[mo.cp_rank], n_random)
    return sorted(set(rows) | set(int(x) for x in extra))


def oracle_rows(c: ZigzagCase, rows: List[int]) -> np.ndarray:
    """Oracle output of the listed local rows, grouped by segment for speed."""
    segs = list(zigzag_meta.segments(c.meta_o))
    q = c.q_local.cpu()
    out = np.zeros((len(rows), q.shape[1], q.shape[2]))
    for _h, b, r0, q_len, kv_len in segs:
        sel = [i for i, r in enumerate(rows) if r0 <= r < r0 + q_len]
        if not sel:
            continue
        loc = [rows[i] - r0 for i in sel]
        out[sel] = oatt.attention_rows(q[[rows[i] for i in sel]], loc, c.k_seqs[b], c.v_seqs[b],
                                       q_len, kv_len, True, c.scale)
    return out
