"""Zigzag context-parallel metadata, plain Python integers (test oracle).

Written from the block layout that the module docstring of [P5] (sglang
zigzag.py source page) prints: every sequence is cut into 2*cp_size blocks
and rank r owns block r (its early block) and block 2*cp_size-1-r (its late
block); after the all-gather the blocks are reranged to their original order.
This module does not transcribe the page's ``build_metadata`` formulas.  It
simulates the layout on the tokens themselves:

  1. cut each sequence into blocks (the one rule taken from ``build_metadata``:
     the remainder of length / 2cp goes one token each to the first blocks);
  2. tag every token with (sequence, block, position);
  3. shard: rank r keeps the tokens of its early blocks of all sequences,
     then those of its late blocks;
  4. all-gather: the ranks' shards one after the other;
and reads every list of ``ZigzagContextParallelMetadata`` off those simulated
buffers (run lengths, run positions, last positions).  The page's own
formulas serve only as pins, in tests/test_oracle_meta.py.

Readings where the page leaves a step open:
  * ``num_tokens`` smaller than the sum of extend lengths is rejected (the page
    only handles a surplus, which goes to the last sequence).
  * Applicability is [P5] ``can_apply``'s condition, read as "every one of the
    2*cp_size blocks of every sequence gets at least one token, on at least
    two ranks"; in addition 0 <= cp_rank < cp_size.
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
    """[P5] can_apply: zigzag needs two or more ranks, and every block of the
    batch and of each sequence must hold at least one token (2*cp_size
    blocks)."""
    nblk = 2 * cp_size
    if cp_size < 2 or num_tokens < nblk:
        return False
    return extend_lens is None or min(int(x) for x in extend_lens) >= nblk


def _blocks_of(length: int, nblocks: int) -> List[int]:
    """[P5] build_metadata: a sequence of ``length`` tokens is cut into
    ``nblocks`` blocks; the remainder ``length mod nblocks`` is spread one
    token each over the first blocks."""
    base, rem = divmod(length, nblocks)
    return [base + (1 if j < rem else 0) for j in range(nblocks)]


def _runs(tags):
    """Maximal runs of equal consecutive tags: [(tag, length), ...]."""
    out = []
    for t in tags:
        if out and out[-1][0] == t:
            out[-1][1] += 1
        else:
            out.append([t, 1])
    return [(t, n) for t, n in out]


def build(cp_size: int, cp_rank: int, num_tokens: int,
          seq_lens: Optional[List[int]] = None,
          extend_lens: Optional[List[int]] = None) -> ZigzagMeta:
    """Metadata of rank ``cp_rank`` for one batch, read off a simulated shard
    and all-gather of the batch's tokens ([P5] module docstring layout)."""
    if not (0 <= cp_rank < cp_size):
        raise NotApplicable(f"cp_rank {cp_rank} outside [0, {cp_size})")
    if extend_lens is None:
        extend_lens = list(seq_lens) if seq_lens else [num_tokens]
    ext = [int(x) for x in extend_lens]
    if not can_apply(cp_size, num_tokens, ext):
        raise NotApplicable("zigzag CP does not apply to this batch")
    seqs = None if seq_lens is None else [int(x) for x in seq_lens]

    # Rows of the batch beyond the sequences' extend tokens are counted as
    # tokens of the last sequence (whose full length grows with them, so its
    # cached prefix stays the same).
    surplus = int(num_tokens) - sum(ext)
    if surplus < 0:
        raise NotApplicable("num_tokens is smaller than the sum of extend lengths")
    ext[-1] += surplus
    if seqs is not None and len(seqs) == len(ext):
        seqs[-1] += surplus

    bs = len(ext)
    nblk = 2 * cp_size
    # Tokens already in the KV cache ahead of each sequence's extend part.
    has_seqs = seqs is not None and len(seqs) == bs
    prefix = [max(seqs[b] - ext[b], 0) if has_seqs else 0 for b in range(bs)]
    blk = [_blocks_of(L, nblk) for L in ext]

    # Every token of the batch, in original order: (sequence, block, position).
    tokens = []
    for b in range(bs):
        t = 0
        for j in range(nblk):
            for _ in range(blk[b][j]):
                tokens.append((b, j, t))
                t += 1

    # Shard: rank r keeps its early block (r) of every sequence, then its
    # late block (2cp-1-r) of every sequence, each in token order.
    of_block = {}
    for tk in tokens:
        of_block.setdefault(tk[:2], []).append(tk)

    def shard(r):
        early = [tk for b in range(bs) for tk in of_block[(b, r)]]
        late = [tk for b in range(bs) for tk in of_block[(b, nblk - 1 - r)]]
        return early, late

    shards = [shard(r) for r in range(cp_size)]
    local = [e + l for e, l in shards]
    gathered = [tk for r in range(cp_size) for tk in local[r]]    # the all-gather, pads left out

    # Chunks: the runs of one (sequence, block) in original token order.
    chunks = _runs((b, j) for b, j, _t in tokens)
    chunk_id = {tag: c for c, (tag, _n) in enumerate(chunks)}
    split_list = [n for _tag, n in chunks]
    per_rank = [len(x) for x in local]
    max_rank_len = [max(per_rank)] * cp_size
    zigzag_index = [chunk_id[tag] for tag, _n in _runs((b, j) for b, j, _t in local[cp_rank])]
    g_runs = _runs((b, j) for b, j, _t in gathered)
    reverse_split_len = [n for _tag, n in g_runs]
    g_pos = {tag: k for k, (tag, _n) in enumerate(g_runs)}
    cp_reverse_index = [g_pos[tag] for tag, _n in chunks]

    # This rank's halves: each local block attends to its sequence up to and
    # including its own last token, after the cached prefix.
    early, late = shards[cp_rank]
    q_prev = [sum(1 for tk in early if tk[0] == b) for b in range(bs)]
    q_next = [sum(1 for tk in late if tk[0] == b) for b in range(bs)]
    kv_len_prev = [prefix[b] + 1 + max(t for bb, _j, t in early if bb == b) for b in range(bs)]
    kv_len_next = [prefix[b] + 1 + max(t for bb, _j, t in late if bb == b) for b in range(bs)]
    cu_prev, cu_next = [0], [0]
    for b in range(bs):
        cu_prev.append(cu_prev[-1] + q_prev[b])
        cu_next.append(cu_next[-1] + q_next[b])

    return ZigzagMeta(
        cp_size=cp_size, cp_rank=cp_rank, bs=bs, extend_lens=ext,
        prefix_offsets=prefix, block_sizes=blk, split_list=split_list,
        per_rank_actual_token=per_rank, max_rank_len=max_rank_len,
        zigzag_index=zigzag_index, cp_reverse_index=cp_reverse_index,
        reverse_split_len=reverse_split_len, kv_len_prev=kv_len_prev,
        kv_len_next=kv_len_next, q_prev=q_prev, q_next=q_next,
        cu_seqlens_q_prev=cu_prev, cu_seqlens_q_next=cu_next,
        total_q_prev_tokens=cu_prev[-1], total_q_next_tokens=cu_next[-1],
        max_seqlen_q_prev=max(q_prev), max_seqlen_q_next=max(q_next),
        total_seq_lens=len(tokens),
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
