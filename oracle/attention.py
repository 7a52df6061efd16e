"""Softmax attention in float64 for zigzag CP and AllGather-KV (test oracle).

Definition used everywhere (one query head h, one segment):
    G       = H_q / H_kv, KV head of query head h is h // G         [P4]
    S       = scale * Q_h K_{h//G}^T                                 scale = 1/sqrt(D) [P4]
    causal: row i of a q_len-row segment sees key j iff j <= i + kv_len - q_len
    P       = exp(S - rowmax) / rowsum
    O_h     = P V_{h//G}

Sources: [P5] run_attention (Q split at total_q_prev_tokens; each half is one
varlen call with its cu_seqlens_q and kv_len; outputs concatenated prev then
next); [P4] (GQA/MQA: H_q must be a multiple of H_kv, else ValueError; each
KV head serves a contiguous group of query heads; scale head_size**-0.5);
[P2] (AllGather-KV: local Q against global K/V, the pad is a strict suffix of
K/V that no query consumes).

Readings: causal alignment is bottom-right (the only
alignment under which the ranks' shares add up to full-sequence causal
attention; tests check that union by brute force); AllGather-KV query rows at
or past ``q_real`` are written as zeros.

Inputs may be any float dtype (bf16 tensors are converted exactly); all
arithmetic is float64 and the result is float64, not rounded.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .zigzag_meta import ZigzagMeta, segments


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (bf16 converts exactly to float64)
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def check_heads(h_q: int, h_kv: int) -> int:
    """[P4]: the query heads must split evenly over the KV heads."""
    if h_kv <= 0 or h_q <= 0 or h_q % h_kv != 0:
        raise ValueError(f"num_heads ({h_q}) must be a multiple of num_kv_heads ({h_kv})")
    return h_q // h_kv


def attention_rows(q: np.ndarray, rows: Sequence[int], k: np.ndarray, v: np.ndarray,
                   q_len: int, kv_len: int, causal: bool, scale: float,
                   block: int = 256) -> np.ndarray:
    """Attention output of the segment rows ``rows`` (segment-local indices).

    q: [n_rows_given, H_q, D] holding exactly the rows listed in ``rows``;
    k, v: [>= kv_len, H_kv, D] -- keys 0..kv_len-1 of the sequence.
    Returns float64 [len(rows), H_q, D].  Rows are processed ``block`` at a
    time only to bound memory."""
    q, k, v = _f64(q), _f64(k)[:kv_len], _f64(v)[:kv_len]
    n, h_q, d = q.shape
    g = check_heads(h_q, k.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((n, h_q, d), dtype=np.float64)
    keys = np.arange(kv_len)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        if causal:
            # bottom-right alignment: row i sees keys up to i + kv_len - q_len
            visible = keys[None, :] <= (rows[r0:r1, None] + kv_len - q_len)
        for h in range(h_q):
            s = scale * (q[r0:r1, h, :] @ k[:, h // g, :].T)
            if causal:
                s = np.where(visible, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            p = np.exp(s - m)
            out[r0:r1, h, :] = (p @ v[:, h // g, :]) / np.sum(p, axis=1, keepdims=True)
    return out


def attention(q, k, v, causal: bool, scale: float, kv_len: Optional[int] = None) -> np.ndarray:
    """All rows of one segment: q [q_len, H_q, D], k/v [kv_len, H_kv, D]."""
    q = _f64(q)
    kv_len = k.shape[0] if kv_len is None else kv_len
    return attention_rows(q, range(q.shape[0]), k, v, q.shape[0], kv_len, causal, scale)


def zigzag_rank(q_local, k_seqs, v_seqs, meta: ZigzagMeta, scale: float) -> np.ndarray:
    """One CP rank's share ([P5] run_attention): both halves, output in local order.

    q_local: [total_q_prev + total_q_next, H_q, D] local rows;
    k_seqs[b], v_seqs[b]: [>= prefix_b + extend_b, H_kv, D] full sequence b."""
    q_local = _f64(q_local)
    out = np.zeros_like(q_local)
    for _half, b, r0, q_len, kv_len in segments(meta):
        out[r0:r0 + q_len] = attention(q_local[r0:r0 + q_len], k_seqs[b], v_seqs[b],
                                       causal=True, scale=scale, kv_len=kv_len)
    return out


def zigzag_rank_rows(q_local, local_rows: Sequence[int], k_seqs, v_seqs,
                     meta: ZigzagMeta, scale: float) -> np.ndarray:
    """Only the listed local rows of one rank's share (for sampling large cases)."""
    segs = list(segments(meta))
    out = []
    for r in local_rows:
        for _half, b, r0, q_len, kv_len in segs:
            if r0 <= r < r0 + q_len:
                qrow = _f64(q_local[r:r + 1])
                out.append(attention_rows(qrow, [r - r0], k_seqs[b], v_seqs[b],
                                          q_len, kv_len, True, scale)[0])
                break
        else:
            raise IndexError(f"local row {r} outside every segment")
    return np.stack(out, axis=0)


def allgather_kv(q_local, k_global, v_global, q_real: int, kv_real: int,
                 scale: float, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """AllGather-KV ([P2]): local Q rows against the real prefix of global K/V.

    Rows < q_real attend (non-causal) to keys 0..kv_real-1; pad rows (>= q_real)
    are zeros.  ``rows`` restricts the output to the listed local rows."""
    q_local = _f64(q_local)
    n = q_local.shape[0]
    rows = list(range(n)) if rows is None else list(rows)
    out = np.zeros((len(rows),) + q_local.shape[1:], dtype=np.float64)
    real = [i for i, r in enumerate(rows) if r < q_real]
    if real:
        sel = [rows[i] for i in real]
        out[real] = attention_rows(q_local[sel], sel, k_global, v_global,
                                   q_len=n, kv_len=kv_real, causal=False, scale=scale)
    return out


def allgather_kv_packed(q_local, k_global, v_global, doc_cu: Sequence[int], q_start: int,
                        scale: float, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """AllGather-KV over a packed global sequence ([P2]: the query ranges of a
    rank's local slice, one per document it covers, and the local query
    boundaries remapped from the global ones).

    The global sequence packs documents back to back: document b holds global
    rows doc_cu[b] .. doc_cu[b+1]-1 (doc_cu[0] = 0) and rows at or past
    doc_cu[-1] are the pad suffix.  Local query row i is global row
    q_start + i; it attends, with no causal mask, to the K/V rows of its own
    document, and its output is zero if it lies in the pad suffix.
    ``rows`` restricts the output to the listed local rows."""
    q_local = _f64(q_local)
    n = q_local.shape[0]
    rows = list(range(n)) if rows is None else list(rows)
    out = np.zeros((len(rows),) + q_local.shape[1:], dtype=np.float64)
    cu = [int(c) for c in doc_cu]
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        sel = [i for i, r in enumerate(rows) if lo <= q_start + r < hi]
        if not sel:
            continue
        local = [rows[i] for i in sel]
        out[sel] = attention_rows(q_local[local], local, k_global[lo:hi], v_global[lo:hi],
                                  q_len=len(local), kv_len=hi - lo, causal=False, scale=scale)
    return out


def default_scale(d: int) -> float:
    """[P4]: softmax scale is head_size ** -0.5."""
    return 1.0 / math.sqrt(d)


def useful_pairs(q_len: int, kv_len: int, causal: bool) -> int:
    """Number of (query, visible key) pairs of one segment and head."""
    if not causal:
        return q_len * kv_len
    off = kv_len - q_len
    return sum(min(kv_len, i + off + 1) for i in range(q_len))
