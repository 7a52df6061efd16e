"""Seeded synthetic inputs for the zigzag CP prefill-attention workloads.

This module only describes workloads and draws random numbers; it holds none
of the method's arithmetic (no block sizes, index maps or attention), so both
the CPU oracle's tests and the HIP path's tests/benchmark can use it.

Recipe (identical everywhere):
  * float data: ``torch.Generator('cpu').manual_seed(seed)``, standard normal
    float32 drawn in the order the caller asks (Q, then K, then V), rounded to
    bfloat16 with round-to-nearest-even (torch ``.to(torch.bfloat16)``);
  * integer structure (sequence and document lengths, page permutations):
    ``numpy.random.default_rng(seed)``.

The workloads are the long-context, varlen and AllGather-KV shapes (single
and packed documents) that the pages' prefill context-parallel discussions
revolve around; the pages print no numeric inputs, so every tensor here is
synthetic.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    causal: bool
    h_q: int
    h_kv: int
    d: int
    page_size: int
    contiguous_kv: bool             # identity page table over a dense [S, H_kv, D]
    cp_size: int = 0                # zigzag workloads
    ranks: Tuple[int, ...] = ()     # zigzag ranks this workload runs
    bs: int = 1
    seq_len: int = 0                # single-sequence zigzag workloads
    varlen: Optional[Tuple[int, int, int]] = None   # (low, high, multiple) for varlen
    # AllGather-KV workload
    kv_total: int = 0               # global K/V rows (real + pad suffix)
    kv_real: int = 0
    ag_degree: int = 0
    ag_rank: int = 0
    kv_heads_variants: Tuple[int, ...] = ()
    packed_docs: Optional[Tuple[int, int]] = None   # (low, high) document lengths of a packed sequence


WORKLOADS = {
    "tiny_cp2_s256": Workload(
        name="tiny_cp2_s256", seed=1, causal=True, h_q=4, h_kv=2, d=64, page_size=16,
        contiguous_kv=True, cp_size=2, ranks=(0, 1), bs=1, seq_len=256),
    "gqa_cp2_s8192": Workload(
        name="gqa_cp2_s8192", seed=2, causal=True, h_q=32, h_kv=4, d=128, page_size=16,
        contiguous_kv=False, cp_size=2, ranks=(0, 1), bs=1, seq_len=8192),
    "varlen_cp4_bs8": Workload(
        name="varlen_cp4_bs8", seed=3, causal=True, h_q=32, h_kv=4, d=128, page_size=16,
        contiguous_kv=False, cp_size=4, ranks=(0, 1, 2, 3), bs=8,
        varlen=(1024, 16384, 8)),
    "long_cp8_s131072_r3": Workload(
        name="long_cp8_s131072_r3", seed=4, causal=True, h_q=64, h_kv=8, d=128, page_size=64,
        contiguous_kv=False, cp_size=8, ranks=(3,), bs=1, seq_len=131072),
    "allgather_kv_s32768": Workload(
        name="allgather_kv_s32768", seed=5, causal=False, h_q=32, h_kv=8, d=128, page_size=64,
        contiguous_kv=True, kv_total=32768, kv_real=30000, ag_degree=4, ag_rank=1,
        kv_heads_variants=(8, 1)),
    "allgather_packed_s32768": Workload(
        name="allgather_packed_s32768", seed=6, causal=False, h_q=32, h_kv=8, d=128, page_size=64,
        contiguous_kv=True, kv_total=32768, kv_real=30000, ag_degree=4, ag_rank=1,
        kv_heads_variants=(8, 1), packed_docs=(500, 8000)),
}

# Order used when workloads are referred to by number (1..5).
WORKLOAD_ORDER = ["tiny_cp2_s256", "gqa_cp2_s8192", "varlen_cp4_bs8",
                  "long_cp8_s131072_r3", "allgather_kv_s32768"]


def sequence_lengths(w: Workload) -> List[int]:
    """Extend lengths of the batch: fixed, or uniform in [low, high] rounded
    down to a multiple (numpy default_rng(seed))."""
    if w.varlen is None:
        return [w.seq_len] * w.bs
    lo, hi, mult = w.varlen
    rng = np.random.default_rng(w.seed)
    u = rng.integers(lo, hi, size=w.bs, endpoint=True)
    return [int(mult * (x // mult)) for x in u]


def packed_doc_cu(w: Workload) -> List[int]:
    """Document boundaries of a packed global sequence: lengths uniform in
    [low, high] (numpy default_rng(seed)) drawn until the next one would pass
    kv_real; the last document takes the remainder, so the real rows total
    exactly kv_real.  Returns [0, cu_1, ..., kv_real]."""
    lo, hi = w.packed_docs
    rng = np.random.default_rng(w.seed)
    cu = [0]
    while True:
        n = int(rng.integers(lo, hi, endpoint=True))
        if cu[-1] + n >= w.kv_real:
            cu.append(w.kv_real)
            return cu
        cu.append(cu[-1] + n)


def page_table(w: Workload, kv_lens: Sequence[int], seed_offset: int = 0):
    """CSR page table for sequences of ``kv_lens`` tokens.

    Each sequence gets ceil(len/page_size) pages.  Contiguous workloads use the
    identity table; paged workloads draw page ids from one shared pool with a
    seeded permutation.  Returns (indptr int32 [bs+1], indices int32, num_pages)."""
    ps = w.page_size
    npages = [(int(n) + ps - 1) // ps for n in kv_lens]
    indptr = np.zeros(len(npages) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    total = int(indptr[-1])
    if w.contiguous_kv:
        indices = np.arange(total, dtype=np.int32)
    else:
        rng = np.random.default_rng(w.seed + 1000 + seed_offset)
        indices = rng.permutation(total).astype(np.int32)
    return indptr, indices, total


def normal_bf16(seed: int, *shapes):
    """Standard-normal float32 tensors drawn in order from one seeded CPU
    generator, each rounded to bfloat16 (round-to-nearest-even)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = []
    for shp in shapes:
        out.append(torch.randn(*shp, generator=g, dtype=torch.float32).to(torch.bfloat16))
    return out
