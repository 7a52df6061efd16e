"""Zigzag context-parallel metadata, plain Python integers (test oracle).

Follows [P5] (sglang zigzag.py source page): the block layout in its module
docstring, ``ZigzagCPStrategy.can_apply`` for validity, and
``ZigzagCPStrategy.build_metadata`` for every list.  Written from the
definitions, step by step, in the pages' names.

Readings where the page leaves a step open:
  * ``num_tokens`` smaller than the sum of extend lengths is rejected (the page
    only handles a surplus, which goes to the last sequence).
  * Validation follows ``can_apply``: cp_size >= 2, num_tokens >= 2*cp_size,
    and every extend length >= 2*cp_size; in addition 0 <= cp_rank < cp_size.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional


class NotApplicable(ValueError):
    """The zigzag strategy does not apply to this batch ([P5] can_apply)."""


@dataclass
class ZigzagMeta:
    cp_size: int
    cp_rank: int
    bs: int
    extend_lens: List[int]
    prefix_offsets: List[int]
    block_sizes: List[List[int]]          # [bs][2*cp_size]
    split_list: List[int]                 # bs*2cp, sequence-major
    per_rank_actual_token: List[int]      # cp_size
    max_rank_len: List[int]               # cp_size copies of the max
    zigzag_index: List[int]               # 2*bs
    cp_reverse_index: List[int]           # bs*2cp
    reverse_split_len: List[int]          # bs*2cp
    kv_len_prev: List[int]                # bs
    kv_len_next: List[int]                # bs
    q_prev: List[int]                     # bs  (actual_seq_q_prev)
    q_next: List[int]                     # bs  (actual_seq_q_next)
    cu_seqlens_q_prev: List[int]          # bs+1
    cu_seqlens_q_next: List[int]          # bs+1
    total_q_prev_tokens: int = 0
    total_q_next_tokens: int = 0
    max_seqlen_q_prev: int = 0
    max_seqlen_q_next: int = 0
    total_seq_lens: int = 0
    extra: dict = field(default_factory=dict)


def can_apply(cp_size: int, num_tokens: int, extend_lens: Optional[List[int]]) -> bool:
    """[P5] can_apply: zigzag CP needs at least two ranks and every sequence
    (and the whole batch) long enough to give each of the 2*cp_size blocks
    at least one token."""
    if cp_size <= 1 or num_tokens < 2 * cp_size:
        return False
    if extend_lens is None:
        return True
    return all(int(x) >= 2 * cp_size for x in extend_lens)


def _blocks_of(length: int, nblocks: int) -> List[int]:
    """[P5] build_metadata: a sequence of ``length`` tokens is cut into
    ``nblocks`` blocks; the remainder ``length mod nblocks`` is spread one
    token each over the first blocks."""
    base, rem = divmod(length, nblocks)
    return [base + (1 if j < rem else 0) for j in range(nblocks)]


def build(cp_size: int, cp_rank: int, num_tokens: int,
          seq_lens: Optional[List[int]] = None,
          extend_lens: Optional[List[int]] = None) -> ZigzagMeta:
    """Metadata of rank ``cp_rank`` for one batch ([P5] build_metadata)."""
    if not (0 <= cp_rank < cp_size):
        raise NotApplicable(f"cp_rank {cp_rank} outside [0, {cp_size})")
    if extend_lens is None:
        extend_lens = list(seq_lens) if seq_lens else [num_tokens]
    ext = [int(x) for x in extend_lens]
    if not can_apply(cp_size, num_tokens, ext):
        raise NotApplicable("zigzag CP does not apply to this batch")
    seqs = None if seq_lens is None else [int(x) for x in seq_lens]

    # Surplus tokens of the batch belong to the last sequence (and lengthen its
    # full length by the same amount, so its cached prefix does not change).
    surplus = int(num_tokens) - sum(ext)
    if surplus < 0:
        raise NotApplicable("num_tokens is smaller than the sum of extend lengths")
    if surplus > 0:
        ext[-1] += surplus
        if seqs is not None and len(seqs) == len(ext):
            seqs[-1] += surplus

    bs = len(ext)
    nblk = 2 * cp_size
    # Tokens already in the KV cache ahead of each sequence's extend part.
    if seqs is not None and len(seqs) == bs:
        prefix = [max(seqs[b] - ext[b], 0) for b in range(bs)]
    else:
        prefix = [0] * bs

    blk = [_blocks_of(L, nblk) for L in ext]
    split_list = [s for b in range(bs) for s in blk[b]]

    # Rank r' holds block r' (its early block) and block 2cp-1-r' (its late
    # block) of every sequence.
    def early(rk: int) -> int:
        return rk

    def late(rk: int) -> int:
        return nblk - 1 - rk

    per_rank = [sum(blk[b][early(rk)] + blk[b][late(rk)] for b in range(bs))
                for rk in range(cp_size)]
    max_rank_len = [max(per_rank)] * cp_size

    # A rank's local rows: the early blocks of all sequences, then the late
    # blocks of all sequences.  Chunk ids index the split_list chunks.
    def local_chunks(rk: int) -> List[int]:
        return ([b * nblk + early(rk) for b in range(bs)] +
                [b * nblk + late(rk) for b in range(bs)])

    zigzag_index = local_chunks(cp_rank)

    # The all-gathered buffer holds the ranks' local rows one rank after the
    # other.  Its chunk k is therefore chunk gathered_order[k] of the original
    # split; cp_reverse_index lists, for each original chunk in order, where
    # it sits in the gathered buffer.
    gathered_order = [c for rk in range(cp_size) for c in local_chunks(rk)]
    where = {c: k for k, c in enumerate(gathered_order)}
    cp_reverse_index = [where[c] for c in range(bs * nblk)]
    reverse_split_len = [split_list[c] for c in gathered_order]

    # Each local block attends to every token of its sequence up to and
    # including itself, after the cached prefix.
    kv_len_prev = [prefix[b] + sum(blk[b][: early(cp_rank) + 1]) for b in range(bs)]
    kv_len_next = [prefix[b] + sum(blk[b][: late(cp_rank) + 1]) for b in range(bs)]
    q_prev = [blk[b][early(cp_rank)] for b in range(bs)]
    q_next = [blk[b][late(cp_rank)] for b in range(bs)]
    cu_prev = [0]
    for x in q_prev:
        cu_prev.append(cu_prev[-1] + x)
    cu_next = [0]
    for x in q_next:
        cu_next.append(cu_next[-1] + x)

    total = sum(ext)
    # The page's own consistency checks.
    assert len(split_list) == bs * nblk
    assert sum(split_list) == total
    assert len(zigzag_index) == 2 * bs
    assert sorted(cp_reverse_index) == list(range(bs * nblk))
    assert sum(per_rank) == total

    return ZigzagMeta(
        cp_size=cp_size, cp_rank=cp_rank, bs=bs, extend_lens=ext,
        prefix_offsets=prefix, block_sizes=blk, split_list=split_list,
        per_rank_actual_token=per_rank, max_rank_len=max_rank_len,
        zigzag_index=zigzag_index, cp_reverse_index=cp_reverse_index,
        reverse_split_len=reverse_split_len, kv_len_prev=kv_len_prev,
        kv_len_next=kv_len_next, q_prev=q_prev, q_next=q_next,
        cu_seqlens_q_prev=cu_prev, cu_seqlens_q_next=cu_next,
        total_q_prev_tokens=cu_prev[-1], total_q_next_tokens=cu_next[-1],
        max_seqlen_q_prev=max(q_prev) if q_prev else 0,
        max_seqlen_q_next=max(q_next) if q_next else 0,
        total_seq_lens=total,
    )


def segments(meta: ZigzagMeta):
    """The 2*bs attention calls of [P5] run_attention, as plain tuples.

    Yields (half, b, q_row0, q_len, kv_len) where ``half`` is "prev" or "next",
    ``q_row0`` is the first local row of the segment (prev halves first, then
    next halves, [P5] run_attention splits Q at total_q_prev_tokens).
    """
    for b in range(meta.bs):
        yield ("prev", b, meta.cu_seqlens_q_prev[b], meta.q_prev[b], meta.kv_len_prev[b])
    for b in range(meta.bs):
        yield ("next", b, meta.total_q_prev_tokens + meta.cu_seqlens_q_next[b],
               meta.q_next[b], meta.kv_len_next[b])
