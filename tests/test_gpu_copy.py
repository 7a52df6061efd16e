"""GPU parity of cp_zigzag_rerange and cp_kv_scatter: bit-exact against the oracle."""

import random

import numpy as np
import pytest
import torch

import context_prefill_attention_amd as cpa
import synth
from oracle import layout, zigzag_meta
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

SENT = np.int16(0x7FC0)   # a bf16 NaN bit pattern, used for pads and untouched memory


def _variants():
    rng = random.Random(17)
    out = [(2, [256], 2 * 64 * 2), (2, [8192], 4 * 128 * 2), (4, synth.sequence_lengths(synth.WORKLOADS["varlen_cp4_bs8"]), 4 * 128 * 2)]
    for _ in range(10):
        cp = rng.choice([2, 3, 4, 5, 8])
        bs = rng.randint(1, 4)
        lens = [rng.randint(2 * cp, 2 * cp * 30 + 11) for _ in range(bs)]
        out.append((cp, lens, rng.choice([16, 48, 256, 2048, 8192])))
    return out


@pytest.mark.parametrize("cp,lens,row_bytes", _variants())
def test_rerange_both_directions_bit_exact(cp, lens, row_bytes):
    total = sum(lens)
    w = row_bytes // 2
    x = np.random.default_rng(len(lens)).integers(-2**15, 2**15, size=(total, w), dtype=np.int16)
    mo = zigzag_meta.build(cp, 0, total, extend_lens=lens)
    meta = cpa.meta_build(cp, 0, lens, device="cuda")
    g_ref = layout.gathered_buffer(x, mo, pad_value=SENT)
    # forward: gathered -> original
    src = torch.from_numpy(g_ref).cuda()
    dst = torch.full((total, w), int(SENT), dtype=torch.int16, device="cuda")
    cpa.zigzag_rerange(meta, src, dst, cpa.GATHERED_TO_ORIG)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), layout.rerange(g_ref, mo))
    # inverse: original -> every rank's shard in the gathered layout; pads untouched
    blank = np.full_like(g_ref, 0x1234)
    dst2 = torch.from_numpy(blank).cuda()
    cpa.zigzag_rerange(meta, torch.from_numpy(x).cuda(), dst2, cpa.ORIG_TO_GATHERED)
    torch.cuda.synchronize()
    assert np.array_equal(dst2.cpu().numpy(), layout.rerange_inverse(x, mo, blank))


@pytest.mark.parametrize("cp,lens,row_bytes", _variants() + [(3, [45, 300], 1), (5, [777, 100], 20), (2, [64], 8)])
def test_rerange_kv_pair_both_directions_bit_exact(cp, lens, row_bytes):
    """cp_zigzag_rerange_kv moves K and V in one launch (rows of any width:
    narrow rows take the one-tensor path twice); both tensors match the
    oracle in both directions, pads untouched."""
    total = sum(lens)
    w = row_bytes // 2 if row_bytes % 2 == 0 else row_bytes
    dt = np.int16 if row_bytes % 2 == 0 else np.int8
    rng = np.random.default_rng(7 + len(lens))
    info = np.iinfo(dt)
    x = rng.integers(info.min, info.max, size=(total, w), dtype=dt)
    y = rng.integers(info.min, info.max, size=(total, w), dtype=dt)
    mo = zigzag_meta.build(cp, 0, total, extend_lens=lens)
    meta = cpa.meta_build(cp, 0, lens, device="cuda")
    pad = dt(0x7F) if dt == np.int8 else SENT
    gx, gy = layout.gathered_buffer(x, mo, pad_value=pad), layout.gathered_buffer(y, mo, pad_value=pad)
    dx = torch.full((total, w), int(pad), dtype=torch.from_numpy(x).dtype, device="cuda")
    dy = torch.full_like(dx, int(pad))
    cpa.zigzag_rerange_kv(meta, torch.from_numpy(gx).cuda(), dx, torch.from_numpy(gy).cuda(), dy,
                          cpa.GATHERED_TO_ORIG)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy(), layout.rerange(gx, mo))
    assert np.array_equal(dy.cpu().numpy(), layout.rerange(gy, mo))
    bx, by = np.full_like(gx, 0x12), np.full_like(gy, 0x21)
    ex, ey = torch.from_numpy(bx).cuda(), torch.from_numpy(by).cuda()
    cpa.zigzag_rerange_kv(meta, torch.from_numpy(x).cuda(), ex, torch.from_numpy(y).cuda(), ey,
                          cpa.ORIG_TO_GATHERED)
    torch.cuda.synchronize()
    assert np.array_equal(ex.cpu().numpy(), layout.rerange_inverse(x, mo, bx))
    assert np.array_equal(ey.cpu().numpy(), layout.rerange_inverse(y, mo, by))


def _narrow_variants():
    rng = random.Random(23)
    out = [(4, [1024, 777, 4093], rb) for rb in (1, 2, 3, 4, 6, 8, 12, 24, 40)]
    for _ in range(6):
        cp = rng.choice([2, 3, 5, 8])
        lens = [rng.randint(2 * cp, 2 * cp * 40 + 13) for _ in range(rng.randint(1, 3))]
        out.append((cp, lens, rng.choice([1, 4, 8, 20])))
    return out


@pytest.mark.parametrize("cp,lens,row_bytes", _narrow_variants())
def test_rerange_narrow_rows_bit_exact(cp, lens, row_bytes):
    """Rows that are not a multiple of 16 bytes (positions, narrow per-token
    tensors), uneven blocks and several sequences, every rank, both directions."""
    total = sum(lens)
    x = np.random.default_rng(row_bytes).integers(0, 256, size=(total, row_bytes), dtype=np.uint8)
    for rank in range(cp):
        mo = zigzag_meta.build(cp, rank, total, extend_lens=lens)
        meta = cpa.meta_build(cp, rank, lens, device="cuda")
        g_ref = layout.gathered_buffer(x, mo, pad_value=0xA5)
        dst = torch.full((total, row_bytes), 0x5A, dtype=torch.uint8, device="cuda")
        cpa.zigzag_rerange(meta, torch.from_numpy(g_ref).cuda(), dst, cpa.GATHERED_TO_ORIG)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy(), layout.rerange(g_ref, mo))
        blank = np.full_like(g_ref, 0x3C)
        dst2 = torch.from_numpy(blank).cuda()
        cpa.zigzag_rerange(meta, torch.from_numpy(x).cuda(), dst2, cpa.ORIG_TO_GATHERED)
        torch.cuda.synchronize()
        assert np.array_equal(dst2.cpu().numpy(), layout.rerange_inverse(x, mo, blank))


@pytest.mark.parametrize("dtype", ["int32", "int64"])
def test_rerange_positions(dtype):
    """Positions of the varlen workload (one int per token) through the
    zigzag layout and back: the gathered shards hold each rank's positions."""
    wl = synth.WORKLOADS["varlen_cp4_bs8"]
    lens = synth.sequence_lengths(wl)
    total = sum(lens)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(dtype)
    mo = zigzag_meta.build(wl.cp_size, 0, total, extend_lens=lens)
    meta = cpa.meta_build(wl.cp_size, 0, lens, device="cuda")
    tdt = getattr(torch, dtype)
    g = torch.full((wl.cp_size * meta.max_rank_len,), -1, dtype=tdt, device="cuda")
    cpa.zigzag_rerange(meta, torch.from_numpy(pos).cuda(), g, cpa.ORIG_TO_GATHERED)
    back = torch.empty(total, dtype=tdt, device="cuda")
    cpa.zigzag_rerange(meta, g, back, cpa.GATHERED_TO_ORIG)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), layout.rerange_inverse(pos, mo, np.full(g.shape, -1, dtype=dtype)))
    assert np.array_equal(back.cpu().numpy(), pos)


def test_rerange_config4_kv_full_size():
    """K and V of the long-context workload: [131072, 8, 128] bf16 each."""
    w = synth.WORKLOADS["long_cp8_s131072_r3"]
    total = w.seq_len
    mo = zigzag_meta.build(w.cp_size, 3, total)
    meta = cpa.meta_build(w.cp_size, 3, [total], device="cuda")
    _, k, v = synth.normal_bf16(w.seed, (1, 1, 1), (total, w.h_kv, w.d), (total, w.h_kv, w.d))
    for t in (k, v):
        xb = gc.bits(t)
        g_ref = layout.gathered_buffer(xb, mo, pad_value=SENT)
        dst = torch.empty((total, w.h_kv, w.d), dtype=torch.bfloat16, device="cuda")
        cpa.zigzag_rerange(meta, torch.from_numpy(g_ref).view(torch.bfloat16).cuda(), dst, cpa.GATHERED_TO_ORIG)
        torch.cuda.synchronize()
        assert np.array_equal(gc.bits(dst), xb)


def test_rerange_kv_pair_config4_full_size():
    """The paired launch on the long-context workload's K and V (the bench step's call)."""
    w = synth.WORKLOADS["long_cp8_s131072_r3"]
    total = w.seq_len
    mo = zigzag_meta.build(w.cp_size, 3, total)
    meta = cpa.meta_build(w.cp_size, 3, [total], device="cuda")
    _, k, v = synth.normal_bf16(w.seed, (1, 1, 1), (total, w.h_kv, w.d), (total, w.h_kv, w.d))
    kb, vb = gc.bits(k), gc.bits(v)
    gk = torch.from_numpy(layout.gathered_buffer(kb, mo, pad_value=SENT)).view(torch.bfloat16).cuda()
    gv = torch.from_numpy(layout.gathered_buffer(vb, mo, pad_value=SENT)).view(torch.bfloat16).cuda()
    dk = torch.empty((total, w.h_kv, w.d), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    cpa.zigzag_rerange_kv(meta, gk, dk, gv, dv, cpa.GATHERED_TO_ORIG)
    torch.cuda.synchronize()
    assert np.array_equal(gc.bits(dk), kb) and np.array_equal(gc.bits(dv), vb)


def _scatter_case(cp, lens, h_kv, d, ps, seq=None, seed=0, spare_pages=5):
    total = sum(lens)
    mo = zigzag_meta.build(cp, 0, total, seq_lens=seq, extend_lens=lens)
    full = [p + e for p, e in zip(mo.prefix_offsets, mo.extend_lens)]
    rng = np.random.default_rng(seed)
    npg = [(n + ps - 1) // ps for n in full]
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    n_pool = int(indptr[-1]) + spare_pages
    indices = rng.permutation(n_pool)[: int(indptr[-1])].astype(np.int32)
    k = rng.integers(-2**15, 2**15, size=(total, h_kv, d), dtype=np.int16)
    v = rng.integers(-2**15, 2**15, size=(total, h_kv, d), dtype=np.int16)
    kg = layout.gathered_buffer(k, mo, pad_value=SENT)
    vg = layout.gathered_buffer(v, mo, pad_value=SENT)
    pool0 = np.full((n_pool, ps, h_kv, d), SENT, dtype=np.int16)
    meta = cpa.meta_build(cp, 0, lens, seq_lens=seq, device="cuda")
    kp = torch.from_numpy(pool0).cuda().view(torch.bfloat16)
    vp = torch.from_numpy(pool0).cuda().view(torch.bfloat16)
    cpa.kv_scatter(meta, torch.from_numpy(kg).cuda().view(torch.bfloat16),
                   torch.from_numpy(vg).cuda().view(torch.bfloat16), kp, vp, ps,
                   torch.from_numpy(indptr).cuda(), torch.from_numpy(indices).cuda())
    torch.cuda.synchronize()
    k_ref = layout.kv_scatter(kg, mo, pool0, indptr, indices, ps)
    v_ref = layout.kv_scatter(vg, mo, pool0, indptr, indices, ps)
    return kp.view(torch.int16).cpu().numpy(), vp.view(torch.int16).cpu().numpy(), k_ref, v_ref


@pytest.mark.parametrize("cp,lens,h_kv,d,ps,seq", [
    (2, [256], 2, 64, 16, None),
    (4, [40, 57, 104], 4, 128, 16, None),
    (3, [31, 20], 1, 128, 1, [40, 20]),          # cached prefix, page size 1
    (8, [200], 8, 128, 64, [264]),
    (2, [13, 15, 16, 17], 2, 64, 4, [13, 20, 16, 30]),
])
def test_scatter_bit_exact_with_sentinels(cp, lens, h_kv, d, ps, seq):
    kp, vp, k_ref, v_ref = _scatter_case(cp, lens, h_kv, d, ps, seq=seq, seed=cp)
    assert np.array_equal(kp, k_ref) and np.array_equal(vp, v_ref)


def test_scatter_config2_and_config3_shapes():
    kp, vp, k_ref, v_ref = _scatter_case(2, [8192], 4, 128, 16, seed=2, spare_pages=0)
    assert np.array_equal(kp, k_ref) and np.array_equal(vp, v_ref)
    lens = synth.sequence_lengths(synth.WORKLOADS["varlen_cp4_bs8"])
    kp, vp, k_ref, v_ref = _scatter_case(4, lens, 4, 128, 16, seed=3)
    assert np.array_equal(kp, k_ref) and np.array_equal(vp, v_ref)


def test_scatter_config4_full_size():
    """K and V of the long-context workload, [131072, 8, 128] each, into 2048
    permuted pages of 64: the launch bench.py times, every slot bit-exact."""
    kp, vp, k_ref, v_ref = _scatter_case(8, [131072], 8, 128, 64, seed=4, spare_pages=0)
    assert np.array_equal(kp, k_ref) and np.array_equal(vp, v_ref)


def test_scatter_then_attention_end_to_end():
    """Gathered K/V -> pool (scatter kernel) -> attention kernel, vs the oracle."""
    import math
    from oracle import attention as oatt
    cp, lens, h_q, h_kv, d, ps = 4, [300, 128], 16, 2, 128, 16
    total = sum(lens)
    qg, kg, vg = synth.normal_bf16(41, (total, h_q, d), (total, h_kv, d), (total, h_kv, d))
    m0 = zigzag_meta.build(cp, 0, total, extend_lens=lens)
    k_gath = layout.gathered_buffer(gc.bits(kg), m0, pad_value=SENT)
    v_gath = layout.gathered_buffer(gc.bits(vg), m0, pad_value=SENT)
    w = synth.Workload(name="e2e", seed=41, causal=True, h_q=h_q, h_kv=h_kv, d=d, page_size=ps,
                       contiguous_kv=False, cp_size=cp)
    indptr, indices, npages = synth.page_table(w, lens)
    ip, ix = torch.from_numpy(indptr).cuda(), torch.from_numpy(indices).cuda()
    kp = torch.zeros(npages, ps, h_kv, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    starts = np.concatenate([[0], np.cumsum(lens)])
    for r in range(cp):
        meta = cpa.meta_build(cp, r, lens, attn_group=h_q // h_kv, device="cuda")
        cpa.kv_scatter(meta, torch.from_numpy(k_gath).cuda().view(torch.bfloat16),
                       torch.from_numpy(v_gath).cuda().view(torch.bfloat16), kp, vp, ps, ip, ix)
        mo = zigzag_meta.build(cp, r, total, extend_lens=lens)
        q_loc = torch.from_numpy(layout.shard(gc.bits(qg), mo)).view(torch.bfloat16)
        out = torch.empty(q_loc.shape, dtype=torch.bfloat16, device="cuda")
        cpa.prefill_attn(q_loc.cuda(), kp, vp, out, meta, 1 / math.sqrt(d), ps, ip, ix)
        torch.cuda.synchronize()
        ref = oatt.zigzag_rank(q_loc, [kg[starts[b]:starts[b + 1]] for b in range(2)],
                               [vg[starts[b]:starts[b + 1]] for b in range(2)], mo, 1 / math.sqrt(d))
        gc.assert_close(out, ref, f"e2e rank {r}")
