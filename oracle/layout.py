"""Zigzag shard / all-gather / rerange / KV-pool scatter as index maps (test oracle).

All operations are bit copies of whole rows; arrays are numpy, row-major with
rows on axis 0 (any trailing shape).  Follows [P5] (sglang zigzag.py source
page): ``shard_hidden_states`` (split by split_list, concatenate in
zigzag_index order), ``_all_gather_reorganized`` (every rank's local rows
zero-padded to max_rank_len, concatenated rank after rank, pads stripped),
``gather_kv_cache`` (split by reverse_split_len, concatenate in
cp_reverse_index order) and ``materialize_full_kv`` (write the full-sequence
K/V rows to the cache slots of the extend tokens).

Readings: the KV pool is ``[num_pages, page_size, ...]``
and the page table is CSR (``page_indptr[bs+1]``, ``page_indices``); extend
token t of sequence b goes to sequence position prefix_b + t.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from .zigzag_meta import ZigzagMeta, build


def _split(x: np.ndarray, sizes: Sequence[int]) -> List[np.ndarray]:
    out, start = [], 0
    for s in sizes:
        out.append(x[start:start + s])
        start += s
    assert start == x.shape[0], "sizes must cover the array exactly"
    return out


def shard(x: np.ndarray, meta: ZigzagMeta) -> np.ndarray:
    """Rank ``meta.cp_rank``'s local rows of ``x`` (x in original token order)."""
    chunks = _split(x, meta.split_list)
    return np.concatenate([chunks[i] for i in meta.zigzag_index], axis=0)


def all_rank_metas(meta: ZigzagMeta) -> List[ZigzagMeta]:
    """The metadata of every rank of the same batch."""
    seq = [p + e for p, e in zip(meta.prefix_offsets, meta.extend_lens)]
    return [build(meta.cp_size, rk, meta.total_seq_lens, seq_lens=seq,
                  extend_lens=meta.extend_lens) for rk in range(meta.cp_size)]


def gathered_buffer(x: np.ndarray, meta: ZigzagMeta, pad_value=0) -> np.ndarray:
    """What the all-gather of every rank's padded local rows produces.

    Rank r' contributes its local rows followed by pad rows up to
    max_rank_len; the ranks follow one another.  ``pad_value`` fills the pad
    rows (the page pads with zeros; tests use NaN to prove pads are never
    read)."""
    metas = all_rank_metas(meta)
    mlen = meta.max_rank_len[0]
    parts = []
    for m in metas:
        loc = shard(x, m)
        pad = np.full((mlen - loc.shape[0],) + x.shape[1:], pad_value, dtype=x.dtype)
        parts.append(np.concatenate([loc, pad], axis=0))
    return np.concatenate(parts, axis=0)


def strip_pads(gathered: np.ndarray, meta: ZigzagMeta) -> np.ndarray:
    """Drop every rank's pad rows from the gathered buffer."""
    mlen = meta.max_rank_len[0]
    return np.concatenate(
        [gathered[rk * mlen: rk * mlen + n] for rk, n in enumerate(meta.per_rank_actual_token)],
        axis=0)


def rerange(gathered: np.ndarray, meta: ZigzagMeta) -> np.ndarray:
    """Gathered (rank-major, padded) rows back to original token order."""
    chunks = _split(strip_pads(gathered, meta), meta.reverse_split_len)
    return np.concatenate([chunks[i] for i in meta.cp_reverse_index], axis=0)


def rerange_inverse(x: np.ndarray, meta: ZigzagMeta, out: np.ndarray) -> np.ndarray:
    """Original-order rows into the gathered layout (every rank's shard at once).

    Pad rows of ``out`` are left as they are."""
    metas = all_rank_metas(meta)
    mlen = meta.max_rank_len[0]
    res = out.copy()
    for rk, m in enumerate(metas):
        loc = shard(x, m)
        res[rk * mlen: rk * mlen + loc.shape[0]] = loc
    return res


def gathered_row_of_token(meta: ZigzagMeta, b: int, t: int) -> int:
    """Row of the gathered buffer that holds extend token t of sequence b.

    Found by walking the blocks of the sequence and the local-row order of the
    owning rank, independently of ``rerange``."""
    cp = meta.cp_size
    nblk = 2 * cp
    blk = meta.block_sizes
    j, start = 0, 0
    while t >= start + blk[b][j]:
        start += blk[b][j]
        j += 1
    owner = j if j < cp else nblk - 1 - j
    if j < cp:   # early block: after the early blocks of sequences < b
        off = sum(blk[bb][owner] for bb in range(b))
    else:        # late block: after all early blocks and the late blocks of sequences < b
        off = (sum(blk[bb][owner] for bb in range(meta.bs)) +
               sum(blk[bb][nblk - 1 - owner] for bb in range(b)))
    return owner * meta.max_rank_len[0] + off + (t - start)


def kv_scatter(gathered: np.ndarray, meta: ZigzagMeta, pool: np.ndarray,
               page_indptr: Sequence[int], page_indices: Sequence[int],
               page_size: int) -> np.ndarray:
    """Write every real token's row of ``gathered`` into its KV-pool slot.

    ``pool`` is ``[num_pages, page_size, ...]``; a copy is returned with only
    the slots of extend tokens written."""
    res = pool.copy()
    for b in range(meta.bs):
        for t in range(meta.extend_lens[b]):
            pos = meta.prefix_offsets[b] + t
            page = page_indices[page_indptr[b] + pos // page_size]
            res[page, pos % page_size] = gathered[gathered_row_of_token(meta, b, t)]
    return res


def pool_to_sequence(pool: np.ndarray, page_indptr: Sequence[int],
                     page_indices: Sequence[int], page_size: int, b: int, n: int) -> np.ndarray:
    """The first ``n`` token rows of sequence b, read out of the KV pool."""
    rows = []
    for pos in range(n):
        rows.append(pool[page_indices[page_indptr[b] + pos // page_size], pos % page_size])
    return np.stack(rows, axis=0) if rows else pool[:0, 0]
