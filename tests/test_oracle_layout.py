"""Pins of the oracle's shard / rerange / scatter index maps."""

import random

import numpy as np

from oracle import layout, zigzag_meta


def _cases(seed=11, n=25):
    rng = random.Random(seed)
    out = []
    for cp in (2, 3, 4, 8):
        for _ in range(n // 4 + 1):
            bs = rng.randint(1, 3)
            lens = [rng.randint(2 * cp, 2 * cp * 4 + 9) for _ in range(bs)]
            surplus = rng.choice([0, 2])
            prefix = [rng.choice([0, 3, 16]) for _ in range(bs)]
            out.append((cp, lens, surplus, prefix))
    return out


def test_rerange_inverts_gather_and_inverse_matches_gathered_buffer():
    for cp, lens, surplus, prefix in _cases():
        total = sum(lens) + surplus
        seq = [p + e for p, e in zip(prefix, lens)]
        m = zigzag_meta.build(cp, 0, total, seq_lens=seq, extend_lens=lens)
        x = np.arange(total * 3, dtype=np.float64).reshape(total, 3)
        g = layout.gathered_buffer(x, m, pad_value=np.nan)
        assert g.shape[0] == cp * m.max_rank_len[0]
        assert np.array_equal(layout.rerange(g, m), x)
        # inverse: original -> gathered, pads untouched (NaN stays NaN)
        blank = np.full_like(g, np.nan)
        inv = layout.rerange_inverse(x, m, blank)
        assert np.array_equal(inv, g, equal_nan=True)
        # every rank's shard sits at its slot in the gathered buffer
        for r, mr in enumerate(layout.all_rank_metas(m)):
            loc = layout.shard(x, mr)
            off = r * m.max_rank_len[0]
            assert np.array_equal(g[off:off + loc.shape[0]], loc)


def test_token_walk_agrees_with_split_concat():
    """Two independent derivations of where token (b, t) sits in the gathered
    buffer: walking the blocks, and the split/concatenate of the page."""
    for cp, lens, surplus, prefix in _cases(seed=3):
        total = sum(lens) + surplus
        m = zigzag_meta.build(cp, 0, total, extend_lens=lens)
        x = np.arange(total)
        g = layout.gathered_buffer(x, m, pad_value=-1)
        start = 0
        for b in range(m.bs):
            for t in range(m.extend_lens[b]):
                assert g[layout.gathered_row_of_token(m, b, t)] == start + t
            start += m.extend_lens[b]


def test_fancy_index_cross_check():
    """Rerange equals numpy fancy indexing by a permutation built from the
    per-rank local orders alone."""
    cp, lens = 4, [40, 24, 72]
    m = zigzag_meta.build(cp, 1, sum(lens), extend_lens=lens)
    x = np.random.default_rng(0).standard_normal((sum(lens), 5))
    g = layout.gathered_buffer(x, m)
    # token ids in the gathered buffer, via the shard of an id vector per rank
    ids = layout.gathered_buffer(np.arange(sum(lens)), m, pad_value=-1)
    perm = np.empty(sum(lens), dtype=np.int64)
    for row, tok in enumerate(ids):
        if tok >= 0:
            perm[tok] = row
    assert np.array_equal(g[perm], x)
    assert np.array_equal(layout.rerange(g, m), g[perm])


def test_scatter_writes_every_real_token_and_nothing_else():
    rng = np.random.default_rng(5)
    for cp, lens, surplus, prefix in _cases(seed=9, n=12):
        total = sum(lens) + surplus
        seq = [p + e for p, e in zip(prefix, lens)]
        m = zigzag_meta.build(cp, 0, total, seq_lens=seq, extend_lens=lens)
        ps = 4
        npages = [(p + e + ps - 1) // ps for p, e in zip(m.prefix_offsets, m.extend_lens)]
        indptr = np.concatenate([[0], np.cumsum(npages)]).astype(np.int64)
        n_pool = int(indptr[-1]) + 3            # a few pages that no sequence owns
        indices = rng.permutation(n_pool)[: int(indptr[-1])]
        x = rng.standard_normal((total, 2, 3))
        g = layout.gathered_buffer(x, m, pad_value=np.nan)
        pool = np.full((n_pool, ps, 2, 3), np.nan)
        out = layout.kv_scatter(g, m, pool, indptr, indices, ps)
        written = np.zeros((n_pool, ps), dtype=bool)
        start = 0
        for b in range(m.bs):
            for t in range(m.extend_lens[b]):
                pos = m.prefix_offsets[b] + t
                pg, sl = indices[indptr[b] + pos // ps], pos % ps
                assert np.array_equal(out[pg, sl], x[start + t])
                written[pg, sl] = True
            start += m.extend_lens[b]
        assert np.all(np.isnan(out[~written]))       # untouched slots keep their sentinel
        assert not np.any(np.isnan(out[written]))    # no pad row was copied
        # reading the pool back gives each sequence's extend rows after its prefix
        start = 0
        for b in range(m.bs):
            seqrows = layout.pool_to_sequence(out, indptr, indices, ps, b,
                                              m.prefix_offsets[b] + m.extend_lens[b])
            assert np.array_equal(seqrows[m.prefix_offsets[b]:], x[start:start + m.extend_lens[b]])
            start += m.extend_lens[b]


def test_strip_pads_tiny_layout_by_hand():
    """cp 2, one sequence of 6 tokens: blocks [2, 2, 1, 1]; rank 0 holds blocks
    0 and 3 (tokens 0, 1, 5), rank 1 blocks 1 and 2 (tokens 2, 3, 4), so
    max_rank_len = 3 and nothing is padded; with 7 tokens (blocks [2, 2, 2, 1])
    rank 0 holds 0, 1, 6 and rank 1 holds 2, 3, 4, 5: rank 0 gets one pad row."""
    m6 = zigzag_meta.build(2, 0, 6)
    x6 = np.arange(6)
    g6 = layout.gathered_buffer(x6, m6, pad_value=-1)
    assert g6.tolist() == [0, 1, 5, 2, 3, 4]
    assert layout.strip_pads(g6, m6).tolist() == [0, 1, 5, 2, 3, 4]
    m7 = zigzag_meta.build(2, 0, 7)
    g7 = layout.gathered_buffer(np.arange(7), m7, pad_value=-1)
    assert g7.tolist() == [0, 1, 6, -1, 2, 3, 4, 5]
    assert layout.strip_pads(g7, m7).tolist() == [0, 1, 6, 2, 3, 4, 5]
