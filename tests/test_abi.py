"""C-ABI tests that run without a GPU: exports, host metadata against the
oracle (bit-exact), internal tables, and fail-closed argument validation."""

import ctypes
import os
import random
import re

import numpy as np
import pytest

import context_prefill_attention_amd as cpa
from oracle import layout, zigzag_meta
from oracle.attention import useful_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


@pytest.fixture(scope="module")
def lib():
    return cpa.load_library()


def test_library_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:int|const char\*)\s+(cp_\w+)\s*\(", text, flags=re.M))
    assert {"cp_meta_build", "cp_allgather_meta_build", "cp_allgather_packed_meta_build",
            "cp_zigzag_rerange", "cp_zigzag_rerange_kv", "cp_kv_scatter",
            "cp_prefill_attn", "cp_prefill_attn_noalloc", "cp_last_error", "cp_version"} <= names
    for n in names:
        assert hasattr(lib, n), n   # ctypes dlsym succeeds


def _cases():
    rng = random.Random(21)
    cases = [(2, [256], None, None), (2, [8192], None, None), (8, [131072], None, None),
             (4, [13, 50, 8], None, None), (2, [13], None, 20), (3, [30, 31, 32], [40, 31, 50], None)]
    for _ in range(40):
        cp = rng.choice([2, 3, 4, 5, 8])
        bs = rng.randint(1, 5)
        lens = [rng.randint(2 * cp, 2 * cp * 9 + 5) for _ in range(bs)]
        seq = None
        if rng.random() < 0.4:
            seq = [e + rng.choice([0, 1, 7, 64]) for e in lens]
        surplus = rng.choice([None, None, sum(lens) + rng.randint(1, 9)])
        cases.append((cp, lens, seq, surplus))
    return cases


# (position, query head) rows one attention work item covers
ROWS_PER_ITEM = 256

LISTS = ["split_list", "zigzag_index", "cp_reverse_index", "reverse_split_len",
         "per_rank_actual_token", "kv_len_prev", "kv_len_next", "q_prev", "q_next",
         "cu_seqlens_q_prev", "cu_seqlens_q_next"]


def _unpack(blob, off, n, fields):
    a = blob[off:off + 4 * fields * n].view(np.int32).reshape(n, fields)
    return a


def test_meta_matches_oracle_bit_exact():
    for cp, lens, seq, ntok in _cases():
        total = ntok if ntok is not None else sum(lens)
        for r in range(cp):
            o = zigzag_meta.build(cp, r, total, seq_lens=seq, extend_lens=lens)
            m = cpa.meta_build(cp, r, lens, seq_lens=seq, num_tokens=total, attn_group=8)
            for name in LISTS:
                oname = {"q_prev": "q_prev", "q_next": "q_next"}.get(name, name)
                assert getattr(m, name) == getattr(o, oname), (name, cp, lens, r)
            assert m.prefix == o.prefix_offsets and m.extend == o.extend_lens
            assert m.max_rank_len == o.max_rank_len[0]
            assert m.total_seq_lens == o.total_seq_lens
            assert m.total_q_prev_tokens == o.total_q_prev_tokens
            assert m.total_q_next_tokens == o.total_q_next_tokens
            assert m.max_seqlen_q_prev == o.max_seqlen_q_prev
            assert m.max_seqlen_q_next == o.max_seqlen_q_next
            assert m.n_local_rows == o.per_rank_actual_token[r]


def test_chunk_table_agrees_with_oracle_token_walk():
    for cp, lens, seq, ntok in _cases()[:20]:
        total = ntok if ntok is not None else sum(lens)
        o = zigzag_meta.build(cp, 0, total, seq_lens=seq, extend_lens=lens)
        m = cpa.meta_build(cp, 0, lens, seq_lens=seq, num_tokens=total)
        ch = _unpack(m.blob, m.off_chunks, m.n_chunks, 8)
        starts = np.concatenate([[0], np.cumsum(o.extend_lens)])
        covered = 0
        for b_, t0, g_row, o_row, n_rows, pos0, _, _ in ch:
            assert o_row == starts[b_] + t0
            assert pos0 == o.prefix_offsets[b_] + t0
            for t in (t0, t0 + n_rows - 1):
                assert layout.gathered_row_of_token(o, b_, t) == g_row + (t - t0)
            covered += n_rows
        assert covered == o.total_seq_lens


@pytest.mark.parametrize("group", [1, 2, 3, 4, 8, 32])
def test_segments_and_work_list(group):
    for cp, lens, seq, ntok in _cases()[:12]:
        total = ntok if ntok is not None else sum(lens)
        o = zigzag_meta.build(cp, 1 % cp, total, seq_lens=seq, extend_lens=lens)
        m = cpa.meta_build(cp, 1 % cp, lens, seq_lens=seq, num_tokens=total, attn_group=group)
        segs = _unpack(m.blob, m.off_segs, m.n_seg, 8)
        osegs = list(zigzag_meta.segments(o))
        assert len(segs) == len(osegs)
        for (q_row0, q_len, q_rows, kv_len, off, page_row, causal, kv_start), (_h, b, r0, ql, kl) in zip(segs, osegs):
            assert (q_row0, q_len, q_rows, kv_len, off, page_row, causal, kv_start) == \
                (r0, ql, ql, kl, kl - ql, b, 1, 0)
        assert m.kv_align == 2**30              # every sequence's keys start its page-table row
        work = _unpack(m.blob, m.off_work, m.n_work, 4)
        tq = ROWS_PER_ITEM // group
        assert m.q_tile == tq
        seen = {s: np.zeros(segs[s][2], dtype=int) for s in range(len(segs))}
        for s, p0, npos, n_tiles in work:
            assert 1 <= npos <= tq
            seen[s][p0:p0 + npos] += 1
            q_len, kv_len = segs[s][1], segs[s][3]
            last = p0 + npos - 1
            # keys the item's last row can see, bottom-right aligned
            kv_end = min(kv_len, last + kv_len - q_len + 1)
            assert n_tiles == -(-kv_end // 64)
        for s in seen:
            assert np.all(seen[s] == 1)       # every row in exactly one item
        nt = work[:, 3]
        assert np.all(nt[:-1] >= nt[1:])      # longest first
        assert m.mean_item_tiles == int(nt.sum()) // len(nt)
        assert not np.any(m.blob[128:128 + 36])   # attention job counters start at zero
        # the visited tiles cover every useful (query, key) pair
        assert sum(useful_pairs(s[1], s[3], True) for s in segs) <= \
            sum(int(w[3]) * 64 * int(w[2]) for w in work)


def test_allgather_meta():
    m = cpa.allgather_meta_build(8192, 8192, 30000, 4)
    assert m.kind == cpa.META_ALLGATHER and m.n_seg == 1 and m.n_local_rows == 8192
    assert m.kv_align == 2**30
    seg = _unpack(m.blob, m.off_segs, 1, 8)[0]
    assert tuple(seg[:7]) == (0, 8192, 8192, 30000, 0, 0, 0)
    work = _unpack(m.blob, m.off_work, m.n_work, 4)
    assert m.n_work == 8192 // (ROWS_PER_ITEM // 4) and np.all(work[:, 3] == -(-30000 // 64))
    assert m.mean_item_tiles == -(-30000 // 64) and not np.any(m.blob[128:128 + 36])
    m = cpa.allgather_meta_build(100, 70, 33, 32)    # pad query rows 70..99
    work = _unpack(m.blob, m.off_work, m.n_work, 4)
    assert work[:, 2].sum() == 100
    for s, p0, npos, nt in work:
        assert nt == (0 if p0 >= 70 else 1)


def _expected_packed_segments(cu, q_start, q_total):
    """Segments the packed AllGather-KV share must have, from its definition:
    one per document that meets the local rows, pad rows joining the last one."""
    segs = []
    q_end = q_start + q_total
    for b in range(len(cu) - 1):
        lo, hi = max(cu[b], q_start), min(cu[b + 1], q_end)
        if lo < hi:
            kv = cu[b + 1] - cu[b]
            segs.append([lo - q_start, hi - lo, hi - lo, kv, kv - (hi - lo), 0, 0, cu[b]])
    if q_end > cu[-1]:
        pad0 = max(cu[-1], q_start) - q_start
        if segs and segs[-1][0] + segs[-1][2] == pad0:
            segs[-1][2] += q_total - pad0
        else:
            segs.append([pad0, 0, q_total - pad0, 0, 0, 0, 0, 0])
    return segs


@pytest.mark.parametrize("cu,q_start,q_total,group", [
    ([0, 3838, 8374, 12757, 15831, 23427, 26695, 30000], 8192, 8192, 4),
    ([0, 3838, 8374, 12757, 15831, 23427, 26695, 30000], 24576, 8192, 32),
    ([0, 37, 137, 142, 442, 506], 432, 144, 4),
    ([0, 37, 137, 137, 442, 506], 0, 144, 1),      # an empty document
    ([0, 100], 150, 50, 8),                         # a slice entirely in the pad suffix
    ([0, 100], 0, 100, 256),
])
def test_allgather_packed_meta(cu, q_start, q_total, group):
    m = cpa.allgather_packed_meta_build(cu, q_start, q_total, group)
    assert m.kind == cpa.META_ALLGATHER and m.n_local_rows == q_total
    segs = _unpack(m.blob, m.off_segs, m.n_seg, 8).tolist()
    assert segs == _expected_packed_segments(cu, q_start, q_total)
    # kv_align: largest power of two (capped at 2^30) dividing every
    # segment's first key position in the page-table row
    starts = [sg[7] for sg in segs if sg[7] != 0]
    align = 2**30
    while any(st % align for st in starts):
        align //= 2
    assert m.kv_align == align
    work = _unpack(m.blob, m.off_work, m.n_work, 4)
    tq = ROWS_PER_ITEM // group
    assert m.q_tile == tq
    covered = np.zeros(q_total, dtype=int)
    for s, p0, npos, n_tiles in work:
        sg = segs[s]
        assert 0 < npos <= tq and p0 + npos <= sg[2]
        covered[sg[0] + p0: sg[0] + p0 + npos] += 1
        assert n_tiles == (0 if p0 >= sg[1] else -(-sg[3] // 64))
    assert np.all(covered == 1)                     # every local row exactly once
    assert list(work[:, 3]) == sorted(work[:, 3], reverse=True)


@pytest.mark.parametrize("args,code", [
    (([0], 0, 8, 4), cpa.CP_ERR_INVALID_ARG),
    (([1, 9], 0, 8, 4), cpa.CP_ERR_INVALID_ARG),
    (([0, 9, 5], 0, 8, 4), cpa.CP_ERR_INVALID_ARG),
    (([0, 0], 0, 8, 4), cpa.CP_ERR_INVALID_ARG),
    (([0, 9], -1, 8, 4), cpa.CP_ERR_INVALID_ARG),
    (([0, 9], 0, 0, 4), cpa.CP_ERR_INVALID_ARG),
    (([0, 9], 2**31 - 4, 8, 4), cpa.CP_ERR_OVERFLOW),
    (([0, 9], 0, 8, 0), cpa.CP_ERR_UNSUPPORTED),
    (([0, 9], 0, 8, 257), cpa.CP_ERR_UNSUPPORTED),
])
def test_allgather_packed_meta_rejections(args, code):
    with pytest.raises(cpa.CpError) as ei:
        cpa.allgather_packed_meta_build(*args)
    assert ei.value.code == code


@pytest.mark.parametrize("kw,code", [
    (dict(cp_size=1, cp_rank=0, extend_lens=[64]), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=2, cp_rank=2, extend_lens=[64]), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=2, cp_rank=-1, extend_lens=[64]), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=4, cp_rank=0, extend_lens=[7]), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=2, cp_rank=0, extend_lens=[8, 3]), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=2, cp_rank=0, extend_lens=[8, 8], num_tokens=15), cpa.CP_ERR_INVALID_ARG),
    (dict(cp_size=2, cp_rank=0, extend_lens=[8], attn_group=257), cpa.CP_ERR_UNSUPPORTED),
    (dict(cp_size=2, cp_rank=0, extend_lens=[2**30, 2**30]), cpa.CP_ERR_OVERFLOW),
])
def test_meta_rejections(kw, code):
    with pytest.raises(cpa.CpError) as ei:
        cpa.meta_build(**kw)
    assert ei.value.code == code
    assert cpa.load_library().cp_last_error()   # a message names the argument


def test_meta_rejection_writes_nothing(lib):
    blob = np.full(4096, 0xAB, dtype=np.uint8)
    cm = cpa.CMeta()
    ext = (ctypes.c_int32 * 1)(3)
    rc = lib.cp_meta_build(2, 0, 1, ext, None, 3, 0, blob.ctypes.data, blob.size, ctypes.byref(cm))
    assert rc == cpa.CP_ERR_INVALID_ARG and np.all(blob == 0xAB)
    # too-small blob: reports the size, writes nothing
    ext = (ctypes.c_int32 * 1)(64)
    small = np.full(64, 0xCD, dtype=np.uint8)
    rc = lib.cp_meta_build(2, 0, 1, ext, None, 64, 8, small.ctypes.data, small.size, ctypes.byref(cm))
    assert rc == cpa.CP_ERR_BUFFER_TOO_SMALL and cm.blob_bytes > 64 and np.all(small == 0xCD)


@pytest.mark.parametrize("args,code", [
    ((0, 0, 10, 4), cpa.CP_ERR_INVALID_ARG),
    ((10, 11, 10, 4), cpa.CP_ERR_INVALID_ARG),
    ((10, 5, 0, 4), cpa.CP_ERR_INVALID_ARG),
    ((10, 5, 10, 0), cpa.CP_ERR_UNSUPPORTED),
])
def test_allgather_meta_rejections(args, code):
    with pytest.raises(cpa.CpError) as ei:
        cpa.allgather_meta_build(*args)
    assert ei.value.code == code


# Fake, never-dereferenced device addresses: every call below must fail on
# the host before it could touch them.  A validation bug would instead launch
# a kernel on them, so these tests only run where no GPU is visible.
FAKE = ctypes.c_void_p(0x10000)
FAKE_MISALIGNED = ctypes.c_void_p(0x10008)


@pytest.fixture
def fake_ok(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake device pointers are passed only where no GPU is visible")
    return lib


def _attn(lib, m, h_q=32, h_kv=4, d=128, scale=0.088, ps=16, q=FAKE, npages=10):
    return lib.cp_prefill_attn(q, FAKE, FAKE, FAKE, h_q, h_kv, d, scale, FAKE, ctypes.byref(m.c),
                               npages, ps, FAKE, FAKE, None)


def test_noalloc_attention_validation_fails_closed(fake_ok):
    """The no-allocation variant validates exactly as cp_prefill_attn, before
    it looks anything up on the device."""
    lib = fake_ok
    m = cpa.meta_build(2, 0, [64], attn_group=8)
    call = lambda h_q=32, h_kv=4, d=128, blob=FAKE: lib.cp_prefill_attn_noalloc(
        FAKE, FAKE, FAKE, FAKE, h_q, h_kv, d, 0.088, blob, ctypes.byref(m.c), 10, 16, FAKE, FAKE, None)
    assert call(h_kv=5) == cpa.CP_ERR_INVALID_ARG and b"multiple" in lib.cp_last_error()
    assert call(d=96) == cpa.CP_ERR_UNSUPPORTED
    assert call(blob=None) == cpa.CP_ERR_INVALID_ARG
    big = cpa.meta_build(2, 0, [64], attn_group=8)
    big.c.n_work = (1 << 23) // 8
    assert lib.cp_prefill_attn_noalloc(FAKE, FAKE, FAKE, FAKE, 64, 8, 128, ctypes.c_float(0.088), FAKE,
                                       ctypes.byref(big.c), 4, 16, FAKE, FAKE, None) == cpa.CP_ERR_OVERFLOW


def test_attention_validation_fails_closed(fake_ok):
    lib = fake_ok
    m = cpa.meta_build(2, 0, [64], attn_group=8)
    assert _attn(lib, m, h_q=32, h_kv=5) == cpa.CP_ERR_INVALID_ARG        # 32/5: not a multiple
    assert b"multiple" in lib.cp_last_error()
    assert _attn(lib, m, h_q=32, h_kv=32) == cpa.CP_ERR_INVALID_ARG       # list built for G=8
    assert _attn(lib, m, d=96) == cpa.CP_ERR_UNSUPPORTED
    m_big = cpa.meta_build(2, 0, [64], attn_group=1)
    assert _attn(lib, m_big, h_q=1 << 18, h_kv=1 << 18) == cpa.CP_ERR_UNSUPPORTED   # 64 rows pass 2^31 bytes
    assert _attn(lib, m, scale=0.0) == cpa.CP_ERR_INVALID_ARG
    assert _attn(lib, m, scale=float("nan")) == cpa.CP_ERR_INVALID_ARG
    assert _attn(lib, m, ps=24) == cpa.CP_ERR_UNSUPPORTED
    assert _attn(lib, m, q=FAKE_MISALIGNED) == cpa.CP_ERR_INVALID_ARG
    assert _attn(lib, m, npages=0) == cpa.CP_ERR_INVALID_ARG
    m0 = cpa.meta_build(2, 0, [64], attn_group=0)
    assert _attn(lib, m0) == cpa.CP_ERR_INVALID_ARG                        # no work list
    bad = cpa.meta_build(2, 0, [64], attn_group=8)
    bad.c.version = 99
    assert _attn(lib, bad) == cpa.CP_ERR_INVALID_ARG
    assert lib.cp_prefill_attn(FAKE, FAKE, FAKE, FAKE, 32, 4, 128, 0.1, None, ctypes.byref(m.c),
                               10, 16, FAKE, FAKE, None) == cpa.CP_ERR_INVALID_ARG


def test_copy_validation_fails_closed(fake_ok):
    lib = fake_ok
    m = cpa.meta_build(2, 0, [64], attn_group=8)
    ag = cpa.allgather_meta_build(64, 64, 64, 8)
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(m.c), 2, FAKE, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, 0, None) == cpa.CP_ERR_INVALID_ARG
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, -4, None) == cpa.CP_ERR_INVALID_ARG
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(m.c), 0, FAKE_MISALIGNED, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(ag.c), 0, FAKE, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    kv = lib.cp_zigzag_rerange_kv
    assert kv(FAKE, ctypes.byref(m.c), 2, FAKE, FAKE, FAKE, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert kv(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, FAKE, FAKE, 0, None) == cpa.CP_ERR_INVALID_ARG
    assert kv(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, None, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert kv(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, FAKE, FAKE_MISALIGNED, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert kv(FAKE, ctypes.byref(ag.c), 0, FAKE, FAKE, FAKE, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert kv(None, ctypes.byref(m.c), 0, FAKE, FAKE, FAKE, FAKE, 256, None) == cpa.CP_ERR_INVALID_ARG
    assert b"NULL" in lib.cp_last_error()
    sc = lib.cp_kv_scatter
    assert sc(FAKE, ctypes.byref(m.c), FAKE, FAKE, FAKE, FAKE, 8, 16, 1, 4, FAKE, FAKE, None) == cpa.CP_ERR_UNSUPPORTED
    assert sc(FAKE, ctypes.byref(m.c), FAKE, FAKE, FAKE, FAKE, 8, 0, 4, 128, FAKE, FAKE, None) == cpa.CP_ERR_INVALID_ARG
    assert sc(FAKE, ctypes.byref(m.c), FAKE, None, FAKE, FAKE, 8, 16, 4, 128, FAKE, FAKE, None) == cpa.CP_ERR_INVALID_ARG
    assert sc(FAKE, ctypes.byref(ag.c), FAKE, FAKE, FAKE, FAKE, 8, 16, 4, 128, FAKE, FAKE, None) == cpa.CP_ERR_INVALID_ARG
    # 2^31-byte rows: 16 rows of 16-byte vectors per workgroup would pass int32
    assert sc(FAKE, ctypes.byref(m.c), FAKE, FAKE, FAKE, FAKE, 8, 16, 1 << 15, 1 << 15, FAKE, FAKE, None) == \
        cpa.CP_ERR_OVERFLOW


def test_grids_past_the_work_item_limit_fail_closed(fake_ok):
    lib = fake_ok
    """HIP refuses a grid of more than 2^32-1 work-items; the calls return
    CP_ERR_OVERFLOW on the host before any launch (no GPU needed)."""
    m = cpa.meta_build(2, 0, [64], attn_group=8)          # 4 chunks of 16 rows
    # rerange: 16-row chunks of 2^33-byte rows = 2^23 16-KiB parts each, 2^25 in all
    assert lib.cp_zigzag_rerange(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, 1 << 33, None) == cpa.CP_ERR_OVERFLOW
    assert b"grid too large" in lib.cp_last_error()
    assert lib.cp_zigzag_rerange_kv(FAKE, ctypes.byref(m.c), 0, FAKE, FAKE, FAKE, FAKE, 1 << 33, None) == \
        cpa.CP_ERR_OVERFLOW
    assert b"grid too large" in lib.cp_last_error()
    # attention: n_work * H_kv workgroups of 512 threads; 2^23 of them is one too many
    big = cpa.meta_build(2, 0, [64], attn_group=8)
    big.c.n_work = (1 << 23) // 8
    rc = lib.cp_prefill_attn(FAKE, FAKE, FAKE, FAKE, 64, 8, 128, ctypes.c_float(0.088), FAKE,
                             ctypes.byref(big.c), 4, 16, FAKE, FAKE, None)
    assert rc == cpa.CP_ERR_OVERFLOW and b"grid too large" in lib.cp_last_error()
    big.c.n_work = (1 << 23) // 8 - 1    # one workgroup under the limit passes validation
    big.c.n_work = 0                     # (and is not launched here: an empty grid returns CP_OK)
    assert lib.cp_prefill_attn(FAKE, FAKE, FAKE, FAKE, 64, 8, 128, ctypes.c_float(0.088), FAKE,
                               ctypes.byref(big.c), 4, 16, FAKE, FAKE, None) == cpa.CP_OK


def test_meta_buffers_are_reused_across_builds():
    """The staging a caller keeps (MetaBuffers) is reused build after build:
    no new buffer once it is large enough, and the device view always holds
    the latest blob.  (On the CPU the 'device' buffer is host memory.)"""
    mb = cpa.MetaBuffers(device="cpu", capacity=256)
    first = cpa.meta_build(8, 3, [131072], attn_group=8, buffers=mb)
    grown = mb.grow_count
    ptr = first.d_blob.data_ptr()
    for r in range(8):
        m = cpa.meta_build(8, r, [131072], attn_group=8, buffers=mb)
        assert m.d_blob.data_ptr() == ptr and mb.grow_count == grown
        assert np.array_equal(m.d_blob.numpy(), m.blob)
    ag = cpa.allgather_meta_build(8192, 8192, 30000, 4, buffers=mb)
    assert ag.d_blob.data_ptr() == ptr and np.array_equal(ag.d_blob.numpy(), ag.blob)
    # a larger blob grows the buffers once, then they are reused again
    big = cpa.meta_build(8, 0, [131072] * 64, attn_group=1, buffers=mb)
    assert mb.grow_count == grown + 1 and mb.capacity >= big.blob.size
    again = cpa.meta_build(8, 0, [131072] * 64, attn_group=1, buffers=mb)
    assert mb.grow_count == grown + 1 and np.array_equal(again.d_blob.numpy(), again.blob)


def test_binding_refuses_cpu_tensors():
    import torch
    m = cpa.meta_build(2, 0, [64], attn_group=2)
    q = torch.zeros(64, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(cpa.CpError):
        cpa.prefill_attn(q, torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16),
                         torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16), q.clone(), m, 0.125, 16,
                         torch.zeros(2, dtype=torch.int32), torch.zeros(4, dtype=torch.int32))


def test_ctypes_meta_mirror_matches_the_c_layout(tmp_path):
    """The binding's CMeta must have cp_meta_t's size and field offsets, as the
    C compiler lays the struct out (a mismatch would corrupt every call)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    names = [f[0] for f in cpa.CMeta._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "cpattn.h"\nint main(void) {\n'
        '  printf("sizeof %zu\\n", sizeof(cp_meta_t));\n'
        + "".join(f'  printf("{n} %zu\\n", offsetof(cp_meta_t, {n}));\n' for n in names)
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    build = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                            "-I", "/opt/rocm/include", str(prog), "-o", str(exe)],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["sizeof"]) == ctypes.sizeof(cpa.CMeta)
    for n in names:
        assert int(out[n]) == getattr(cpa.CMeta, n).offset, n
