"""Pins of the oracle's fp64 attention: brute force, a library special case,
closed forms and invariances."""

import math
import random

import numpy as np
import pytest
import torch

import oracle.attention as oatt
from oracle import layout, zigzag_meta


def _textbook_causal(q, k, v, scale):
    """Full-sequence causal attention written as a per-row loop with math.exp
    (tiny inputs only).  q [L, Hq, D], k/v [L, Hkv, D]; head h uses KV head
    h // (Hq/Hkv)."""
    L, hq, d = q.shape
    g = hq // k.shape[1]
    out = np.zeros((L, hq, d))
    for h in range(hq):
        for i in range(L):
            s = [scale * float(np.dot(q[i, h], k[j, h // g])) for j in range(i + 1)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            z = sum(w)
            for j in range(i + 1):
                out[i, h] += (w[j] / z) * v[j, h // g]
    return out


def _union_over_ranks(cp, lens, hq, hkv, d, seed, prefix=None):
    """Every rank's share, gathered rank-major and reranged, against the
    full-sequence textbook result."""
    rng = np.random.default_rng(seed)
    prefix = prefix or [0] * len(lens)
    full = [p + e for p, e in zip(prefix, lens)]
    qs = [rng.standard_normal((n, hq, d)) for n in full]
    ks = [rng.standard_normal((n, hkv, d)) for n in full]
    vs = [rng.standard_normal((n, hkv, d)) for n in full]
    scale = 1 / math.sqrt(d)
    # extend rows of every sequence, concatenated in original order
    q_ext = np.concatenate([q[p:] for q, p in zip(qs, prefix)], axis=0)
    m0 = zigzag_meta.build(cp, 0, sum(lens), seq_lens=full, extend_lens=lens)
    outs = []
    for m in layout.all_rank_metas(m0):
        q_loc = layout.shard(q_ext, m)
        outs.append(oatt.zigzag_rank(q_loc, ks, vs, m, scale))
    o_gath = np.concatenate(
        [np.concatenate([o, np.zeros((m0.max_rank_len[0] - o.shape[0],) + o.shape[1:])])
         for o in outs], axis=0)
    o_orig = layout.rerange(o_gath, m0)
    ref = np.concatenate([_textbook_causal(q, k, v, scale)[p:]
                          for q, k, v, p in zip(qs, ks, vs, prefix)], axis=0)
    return o_orig, ref


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_union_of_ranks_equals_full_causal_attention(cp):
    rng = random.Random(cp)
    for trial in range(3):
        bs = rng.randint(1, 3)
        lens = [rng.randint(2 * cp, 2 * cp + 11) for _ in range(bs)]   # uneven blocks included
        hkv = rng.choice([1, 2])
        got, ref = _union_over_ranks(cp, lens, 2 * hkv if trial else hkv, hkv, 4, seed=trial)
        assert np.max(np.abs(got - ref)) < 1e-12


def test_union_with_cached_prefix():
    got, ref = _union_over_ranks(2, [9, 12], 2, 1, 4, seed=4, prefix=[5, 0])
    assert np.max(np.abs(got - ref)) < 1e-12


def test_planted_top_left_alignment_is_caught(monkeypatch):
    """A plausible mistake -- aligning each half's causal mask top-left instead
    of bottom-right -- must fail the brute-force union check."""
    orig = oatt.attention_rows

    def top_left(q, rows, k, v, q_len, kv_len, causal, scale, block=256):
        return orig(q, rows, k, v, kv_len, kv_len, causal, scale, block)  # offset 0

    monkeypatch.setattr(oatt, "attention_rows", top_left)
    got, ref = _union_over_ranks(2, [16], 2, 1, 4, seed=1)
    assert np.max(np.abs(got - ref)) > 1e-3


def test_matches_torch_sdpa_float64():
    """Library special case: torch's scaled_dot_product_attention in float64
    with an explicit bottom-right boolean mask (causal) or none."""
    rng = np.random.default_rng(3)
    for q_len, kv_len, hq, hkv, causal in [(7, 19, 4, 2, True), (16, 16, 2, 2, True),
                                           (5, 33, 8, 1, False), (12, 40, 4, 4, False)]:
        d = 8
        q = rng.standard_normal((q_len, hq, d))
        k = rng.standard_normal((kv_len, hkv, d))
        v = rng.standard_normal((kv_len, hkv, d))
        scale = 0.37
        got = oatt.attention(q, k, v, causal=causal, scale=scale)
        g = hq // hkv
        tq = torch.from_numpy(q).permute(1, 0, 2)
        tk = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
        tv = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
        mask = None
        if causal:
            i = torch.arange(q_len)[:, None]
            j = torch.arange(kv_len)[None, :]
            mask = j <= i + (kv_len - q_len)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
        assert np.max(np.abs(got - ref)) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(8)
    d, hq, hkv = 8, 4, 2
    k = rng.standard_normal((20, hkv, d))
    v = rng.standard_normal((20, hkv, d))
    # the first token of a sequence sees only itself: O = V_0
    q = rng.standard_normal((20, hq, d))
    o = oatt.attention(q, k, v, causal=True, scale=0.5)
    for h in range(hq):
        assert np.allclose(o[0, h], v[0, h // 2], atol=1e-14)
    # Q = 0: uniform weights over the visible prefix
    o = oatt.attention(np.zeros((6, hq, d)), k, v, causal=True, scale=0.5, kv_len=15)
    for i in range(6):
        vis = i + 15 - 6 + 1
        for h in range(hq):
            assert np.allclose(o[i, h], v[:vis, h // 2].mean(axis=0), atol=1e-13)
    # all keys equal: uniform weights as well
    keq = np.repeat(k[:1], 20, axis=0)
    o = oatt.attention(q[:6], keq, v, causal=False, scale=0.5, kv_len=11)
    for h in range(hq):
        assert np.allclose(o[:, h], np.broadcast_to(v[:11, h // 2].mean(axis=0), (6, d)), atol=1e-13)


def test_head_mappings():
    rng = np.random.default_rng(2)
    d = 8
    q = rng.standard_normal((9, 8, d))
    k = rng.standard_normal((14, 2, d))
    v = rng.standard_normal((14, 2, d))
    # GQA == MHA with each KV head repeated over a consecutive group of query heads
    o = oatt.attention(q, k, v, causal=True, scale=0.3)
    o_mha = oatt.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), causal=True, scale=0.3)
    assert np.max(np.abs(o - o_mha)) < 1e-14
    # MHA is the identity mapping: head h alone gives the same as head h in the batch
    km = np.repeat(k, 4, axis=1)
    vm = np.repeat(v, 4, axis=1)
    for h in range(8):
        oh = oatt.attention(q[:, h:h + 1], km[:, h:h + 1], vm[:, h:h + 1], causal=True, scale=0.3)
        assert np.max(np.abs(oh[:, 0] - o_mha[:, h])) < 1e-14
    # MQA: one KV head serves every query head
    o1 = oatt.attention(q, k[:, :1], v[:, :1], causal=False, scale=0.3)
    for h in range(8):
        oh = oatt.attention(q[:, h:h + 1], k[:, :1], v[:, :1], causal=False, scale=0.3)
        assert np.max(np.abs(oh[:, 0] - o1[:, h])) < 1e-14
    # a plausible mistake, interleaved groups (h % H_kv), differs
    k_il = k[:, [h % 2 for h in range(8)]]
    v_il = v[:, [h % 2 for h in range(8)]]
    o_il = oatt.attention(q, k_il, v_il, causal=True, scale=0.3)
    assert np.max(np.abs(o_il - o)) > 1e-3


@pytest.mark.parametrize("hkv,ok", [(32, True), (8, True), (1, True), (5, False)])
def test_head_ratio_contract(hkv, ok):
    """The GQA report's matrix: 32/32, 32/8, 32/1 accepted; 32/5 rejected."""
    if ok:
        assert oatt.check_heads(32, hkv) == 32 // hkv
    else:
        with pytest.raises(ValueError):
            oatt.check_heads(32, hkv)


def test_key_shift_invariance():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((10, 2, 8))
    k = rng.standard_normal((25, 1, 8))
    v = rng.standard_normal((25, 1, 8))
    c = rng.standard_normal(8) * 3
    o1 = oatt.attention(q, k, v, causal=True, scale=0.4)
    o2 = oatt.attention(q, k + c, v, causal=True, scale=0.4)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_row_sampling_equals_full_share():
    rng = np.random.default_rng(6)
    lens = [24, 40]
    m = zigzag_meta.build(2, 1, sum(lens), extend_lens=lens)
    qloc = rng.standard_normal((m.per_rank_actual_token[1], 4, 8))
    ks = [rng.standard_normal((n, 2, 8)) for n in lens]
    vs = [rng.standard_normal((n, 2, 8)) for n in lens]
    full = oatt.zigzag_rank(qloc, ks, vs, m, 0.3)
    rows = [0, 5, 13, 20, 31]
    assert np.max(np.abs(oatt.zigzag_rank_rows(qloc, rows, ks, vs, m, 0.3) - full[rows])) < 1e-14


def test_allgather_kv_pad_suffix_and_pad_rows():
    """AllGather-KV: K/V rows past kv_real (NaN here) are never consumed;
    local query rows past q_real are zeros; real rows equal plain attention
    over the real prefix."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((12, 4, 8))
    k = rng.standard_normal((40, 2, 8))
    v = rng.standard_normal((40, 2, 8))
    k[33:] = np.nan
    v[33:] = np.nan
    o = oatt.allgather_kv(q, k, v, q_real=9, kv_real=33, scale=0.3)
    assert not np.any(np.isnan(o))
    assert np.all(o[9:] == 0)
    ref = oatt.attention(q[:9], k[:33], v[:33], causal=False, scale=0.3)
    assert np.max(np.abs(o[:9] - ref)) < 1e-14
    sub = oatt.allgather_kv(q, k, v, q_real=9, kv_real=33, scale=0.3, rows=[1, 10, 4])
    assert np.array_equal(sub, o[[1, 10, 4]])


def test_useful_pairs_closed_forms():
    assert oatt.useful_pairs(5, 5, True) == 15
    assert oatt.useful_pairs(4, 10, True) == sum(range(7, 11))
    assert oatt.useful_pairs(8192, 30000, False) == 8192 * 30000


def _packed_case(rng, lens, pad, hq, hkv, d=8):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    total = cu[-1] + pad
    qg = rng.standard_normal((total, hq, d))
    k = rng.standard_normal((total, hkv, d))
    v = rng.standard_normal((total, hkv, d))
    k[cu[-1]:] = np.nan      # the pad suffix is never consumed
    v[cu[-1]:] = np.nan
    return cu, qg, k, v


def test_allgather_packed_matches_sdpa_block_diagonal_float64():
    """Library special case: attention over the whole packed sequence with a
    block-diagonal mask (a row sees exactly its own document's keys), by
    torch's scaled_dot_product_attention in float64, restricted to each
    rank's local slice of rows."""
    rng = np.random.default_rng(11)
    for lens, pad, hq, hkv, a in [([5, 9, 3, 7], 8, 4, 2, 4), ([20], 4, 2, 1, 2), ([1, 1, 6, 2, 2], 0, 6, 3, 3)]:
        cu, qg, k, v = _packed_case(rng, lens, pad, hq, hkv)
        total = qg.shape[0]
        real = cu[-1]
        doc = np.searchsorted(np.asarray(cu), np.arange(real), side="right") - 1
        g = hq // hkv
        tq = torch.from_numpy(qg[:real]).permute(1, 0, 2)
        tk = torch.from_numpy(np.repeat(k[:real], g, axis=1)).permute(1, 0, 2)
        tv = torch.from_numpy(np.repeat(v[:real], g, axis=1)).permute(1, 0, 2)
        mask = torch.from_numpy(doc[:, None] == doc[None, :])
        full = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=mask, scale=0.41).permute(1, 0, 2).numpy()
        share = -(-total // a)
        for r in range(a):
            q0, q1 = r * share, min(total, (r + 1) * share)
            got = oatt.allgather_kv_packed(qg[q0:q1], k, v, cu, q0, scale=0.41)
            assert not np.any(np.isnan(got))
            for i in range(q1 - q0):
                if q0 + i < real:
                    assert np.max(np.abs(got[i] - full[q0 + i])) < 1e-12
                else:
                    assert np.all(got[i] == 0)


def test_allgather_packed_closed_forms_and_special_cases():
    rng = np.random.default_rng(12)
    # documents of one token: each row sees only itself, so O = that row's V
    cu, qg, k, v = _packed_case(rng, [1] * 6, 2, 4, 2)
    o = oatt.allgather_kv_packed(qg[2:8], k, v, cu, 2, scale=0.5)
    g = 2
    for i in range(4):
        for h in range(4):
            assert np.allclose(o[i, h], v[2 + i, h // g], atol=1e-15, rtol=0)
    assert np.all(o[4:] == 0)
    # one document starting at row 0 is the single-range AllGather-KV share
    cu, qg, k, v = _packed_case(rng, [30], 6, 4, 4)
    a = oatt.allgather_kv_packed(qg[10:36], k, v, cu, 10, scale=0.3)
    b = oatt.allgather_kv(qg[10:36], k, v, q_real=20, kv_real=30, scale=0.3)
    assert np.max(np.abs(a - b)) < 1e-14
    # row sampling gives the same rows
    sub = oatt.allgather_kv_packed(qg[10:36], k, v, cu, 10, scale=0.3, rows=[25, 3, 19])
    assert np.array_equal(sub, a[[25, 3, 19]])


def test_allgather_packed_document_order_invariance():
    """Moving a document elsewhere in the packing moves its outputs with it and
    changes nothing else (documents do not see each other)."""
    rng = np.random.default_rng(13)
    lens = [4, 7, 5]
    cu, qg, k, v = _packed_case(rng, lens, 0, 2, 1)
    o = oatt.allgather_kv_packed(qg, k, v, cu, 0, scale=0.7)
    order = [2, 0, 1]
    segs = [slice(cu[b], cu[b + 1]) for b in order]
    q2, k2, v2 = (np.concatenate([x[s] for s in segs]) for x in (qg, k, v))
    cu2 = [0]
    for b in order:
        cu2.append(cu2[-1] + lens[b])
    o2 = oatt.allgather_kv_packed(q2, k2, v2, cu2, 0, scale=0.7)
    assert np.max(np.abs(o2 - np.concatenate([o[s] for s in segs]))) < 1e-14


def test_default_scale_values():
    """head_size ** -0.5 ([P4]) at head sizes where it is exact in binary."""
    assert oatt.default_scale(64) == 0.125
    assert oatt.default_scale(16) == 0.25
    assert oatt.default_scale(256) == 0.0625
    assert abs(oatt.default_scale(128) ** 2 * 128 - 1.0) < 1e-15


def test_softmax_closed_form_at_large_scores():
    """Two keys whose scores are about 800 and differ by ln 3: the weights are
    exactly 1/4 and 3/4 (softmax depends on score differences only), so
    O = (v0 + 3 v1) / 4.  exp(800) overflows float64, so the row maximum
    must be subtracted before exponentiating."""
    d = 4
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, d))
    k[0, 0, 0] = 800.0
    k[1, 0, 0] = 800.0 + math.log(3.0)
    v = np.array([[[1.0, 0.0, 2.0, -4.0]], [[5.0, 4.0, -2.0, 0.0]]])
    out = oatt.attention(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(out[0, 0], (v[0, 0] + 3 * v[1, 0]) / 4, rtol=0, atol=1e-12)
