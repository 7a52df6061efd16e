"""Pins of the oracle's zigzag metadata against what the pages and arithmetic fix."""

import itertools
import os
import random

import pytest

from oracle import layout, zigzag_meta
from oracle.attention import useful_pairs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    lines = []
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                lines.append(ln)
    return lines


def test_printed_cp4_block_layout():
    """Module docstring of the zigzag.py page: cp=4 block ownership and the
    gathered order b0 b7 b1 b6 b2 b5 b3 b4, reranged back to b0..b7."""
    g = _read_golden("zigzag_cp4_layout.txt")
    cp = int(g[0].split()[1])
    owned = {}
    for ln in g[1:1 + cp]:
        parts = ln.split()
        owned[int(parts[1])] = [int(parts[3]), int(parts[4])]
    gathered = [int(x) for x in g[1 + cp].split()[1:]]
    reranged = [int(x) for x in g[2 + cp].split()[1:]]
    for L in (8, 64, 8 * 37):
        for r in range(cp):
            m = zigzag_meta.build(cp, r, L)
            assert m.zigzag_index == owned[r]
        # tag every token with its block id and run it through the gathered buffer
        import numpy as np
        b = L // (2 * cp)
        x = np.repeat(np.arange(2 * cp), b)
        m = zigzag_meta.build(cp, 0, L)
        gbuf = layout.gathered_buffer(x, m, pad_value=-1)
        blocks_in_gathered = [int(v) for v in gbuf[::b]]
        assert blocks_in_gathered == gathered
        back = layout.rerange(gbuf, m)
        assert [int(v) for v in back[::b]] == reranged


def test_hand_derived_small_cases():
    g = _read_golden("zigzag_small_cases.txt")
    vals = {}
    case = None
    for ln in g:
        if ln.startswith("case"):
            case = ln.split()[1]
            continue
        key, _, rest = ln.partition(":")
        vals[(case, key.strip())] = [int(x) for x in rest.split()]
    m0 = zigzag_meta.build(2, 0, 16, extend_lens=[8, 8])
    m1 = zigzag_meta.build(2, 1, 16, extend_lens=[8, 8])
    assert m0.zigzag_index == vals[("A", "zigzag_index rank 0")]
    assert m1.zigzag_index == vals[("A", "zigzag_index rank 1")]
    assert m0.cp_reverse_index == vals[("A", "cp_reverse_index")]
    assert m1.cp_reverse_index == vals[("A", "cp_reverse_index")]
    mb = zigzag_meta.build(2, 0, 13)
    assert mb.block_sizes[0] == vals[("B", "block_sizes")]
    assert [mb.kv_len_prev[0]] == vals[("B", "kv_len_prev")]
    assert [mb.kv_len_next[0]] == vals[("B", "kv_len_next")]
    assert [mb.q_prev[0]] == vals[("B", "q_prev")]
    assert [mb.q_next[0]] == vals[("B", "q_next")]
    mc = zigzag_meta.build(2, 1, 13)
    assert [mc.kv_len_prev[0]] == vals[("C", "kv_len_prev")]
    assert [mc.kv_len_next[0]] == vals[("C", "kv_len_next")]
    assert [mc.q_prev[0]] == vals[("C", "q_prev")]
    assert [mc.q_next[0]] == vals[("C", "q_next")]


@pytest.mark.parametrize("cp", [2, 3, 4, 8])
def test_equal_blocks_closed_forms(cp):
    """With equal blocks of b tokens: kv_len_prev=(r+1)b, kv_len_next=(2cp-r)b,
    and every rank owns the same number of causal (query, key) pairs,
    b^2(2cp-1) + b(b+1) -- the load balance zigzag is for."""
    for b in (1, 3, 16):
        L = 2 * cp * b
        for r in range(cp):
            m = zigzag_meta.build(cp, r, L)
            assert m.kv_len_prev == [(r + 1) * b]
            assert m.kv_len_next == [(2 * cp - r) * b]
            assert m.q_prev == [b] and m.q_next == [b]
            assert m.per_rank_actual_token == [2 * b] * cp
            pairs = (useful_pairs(b, (r + 1) * b, True) +
                     useful_pairs(b, (2 * cp - r) * b, True))
            assert pairs == b * b * (2 * cp - 1) + b * (b + 1)


def _closed_form_reverse_index(cp, bs):
    """cp_reverse_index written as a closed form: early block k of sequence b
    is rank k's chunk b, i.e. gathered chunk b + 2*bs*k; late block 2cp-1-k is
    rank k's chunk bs+b."""
    out = []
    for b in range(bs):
        out += [b + 2 * bs * k for k in range(cp)]
        out += [(2 * cp - 1) * bs + b - 2 * bs * k for k in range(cp)]
    return out


def _random_batch(rng, cp):
    bs = rng.randint(1, 4)
    lens = [rng.randint(2 * cp, 2 * cp * 5 + 7) for _ in range(bs)]
    return bs, lens


def test_invariants_and_closed_form_reverse_index():
    rng = random.Random(7)
    for cp in (2, 3, 4, 5, 8):
        for _ in range(20):
            bs, lens = _random_batch(rng, cp)
            surplus = rng.choice([0, 0, 3])
            prefix = [rng.choice([0, 0, 5, 17]) for _ in range(bs)]
            seq = [p + e for p, e in zip(prefix, lens)]
            for r in range(cp):
                m = zigzag_meta.build(cp, r, sum(lens) + surplus, seq_lens=seq, extend_lens=lens)
                nblk = 2 * cp
                assert len(m.split_list) == bs * nblk
                assert sum(m.split_list) == sum(lens) + surplus
                assert m.extend_lens[-1] == lens[-1] + surplus
                assert m.prefix_offsets == prefix
                assert sorted(m.cp_reverse_index) == list(range(bs * nblk))
                assert m.cp_reverse_index == _closed_form_reverse_index(cp, bs)
                assert sum(m.per_rank_actual_token) == m.total_seq_lens
                assert m.max_rank_len == [max(m.per_rank_actual_token)] * cp
                # block sizes differ by at most one, larger blocks first
                for blk in m.block_sizes:
                    assert max(blk) - min(blk) <= 1 and blk == sorted(blk, reverse=True)
                # kv lengths: each half sees its own block and everything before it
                for b in range(bs):
                    assert m.kv_len_prev[b] - prefix[b] == sum(m.block_sizes[b][:r + 1])
                    assert m.kv_len_next[b] - prefix[b] == m.extend_lens[b] - sum(m.block_sizes[b][2 * cp - r:])
                assert m.cu_seqlens_q_prev[-1] + m.cu_seqlens_q_next[-1] == m.per_rank_actual_token[r]


def test_surplus_goes_to_last_sequence():
    m = zigzag_meta.build(2, 0, 40, extend_lens=[8, 12])
    assert m.extend_lens == [8, 32]
    m = zigzag_meta.build(2, 0, 40, seq_lens=[10, 20], extend_lens=[8, 12])
    assert m.extend_lens == [8, 32] and m.prefix_offsets == [2, 8]


@pytest.mark.parametrize("args", [
    dict(cp_size=1, cp_rank=0, num_tokens=64),             # one rank: not CP
    dict(cp_size=2, cp_rank=2, num_tokens=64),             # rank out of range
    dict(cp_size=4, cp_rank=0, num_tokens=7),              # fewer tokens than blocks
    dict(cp_size=2, cp_rank=0, num_tokens=10, extend_lens=[3, 7]),  # a sequence < 2cp
    dict(cp_size=2, cp_rank=0, num_tokens=10, extend_lens=[8, 8]),  # fewer tokens than extends
])
def test_rejections(args):
    with pytest.raises(zigzag_meta.NotApplicable):
        zigzag_meta.build(**args)


def test_zigzag_order_is_not_rank_major():
    """Reading the gathered buffer as if it were already in token order gives
    the wrong rows for every cp >= 2 (the rank-major vs zigzag pitfall the
    prefill-CP E2E pull request runs into)."""
    import numpy as np
    for cp in (2, 3, 4, 8):
        L = 2 * cp * 3
        x = np.arange(L)
        m = zigzag_meta.build(cp, 0, L)
        g = layout.gathered_buffer(x, m)
        assert not np.array_equal(g, x)
        assert np.array_equal(layout.rerange(g, m), x)
    # cp=2: the gathered block order is b0 b3 b1 b2
    m = zigzag_meta.build(2, 0, 8)
    g = layout.gathered_buffer(np.arange(8), m)
    assert [int(v) for v in g[::2] // 2] == [0, 3, 1, 2]


def test_segments_cover_local_rows_in_order():
    for cp, lens in itertools.product((2, 4), ([16], [16, 24, 40])):
        for r in range(cp):
            m = zigzag_meta.build(cp, r, sum(lens), extend_lens=lens)
            segs = list(zigzag_meta.segments(m))
            assert len(segs) == 2 * len(lens)
            row = 0
            for _h, _b, r0, q_len, _kv in segs:
                assert r0 == row
                row += q_len
            assert row == m.per_rank_actual_token[r]


@pytest.mark.parametrize("cp,ntok,lens,ok", [
    (2, 4, [4], True),            # exactly 2*cp tokens: one token per block
    (2, 3, [3], False),           # one block would be empty
    (4, 64, [8, 56], True),
    (4, 64, [7, 57], False),      # the first sequence is one token short
    (1, 100, [100], False),       # a single rank is not context parallel
    (3, 6, None, True),           # no per-sequence lengths: only the batch total counts
    (3, 5, None, False),
])
def test_can_apply_boundaries(cp, ntok, lens, ok):
    """The zigzag strategy's applicability ([P5] can_apply) at its exact
    boundaries: every one of the 2*cp blocks must get at least one token."""
    assert zigzag_meta.can_apply(cp, ntok, lens) is ok


def _page_formulas(cp, r, lens, prefix):
    """The lists as the build_metadata formulas of the sglang zigzag.py
    source page state them (block sizes per sequence; per-rank counts from
    blocks r and 2cp-1-r; the kept chunk ids as two strided ranges; the
    gathered chunk sizes rank by rank; kv lengths as prefix sums of block
    sizes).  Used only to pin the oracle, which simulates the token walk."""
    n = 2 * cp
    bs = len(lens)
    blk = [[L // n + (1 if j < L % n else 0) for j in range(n)] for L in lens]
    per_rank = [sum(bb[k] + bb[n - 1 - k] for bb in blk) for k in range(cp)]
    zz = list(range(r, r + bs * n, n)) + list(range(n - r - 1, bs * n, n))
    rsl = []
    for k in range(cp):
        rsl += [blk[b][k] for b in range(bs)] + [blk[b][n - 1 - k] for b in range(bs)]
    kvp = [prefix[b] + sum(blk[b][:r + 1]) for b in range(bs)]
    kvn = [prefix[b] + sum(blk[b][:n - r]) for b in range(bs)]
    return dict(split_list=[x for bb in blk for x in bb], per_rank_actual_token=per_rank,
                zigzag_index=zz, reverse_split_len=rsl, kv_len_prev=kvp, kv_len_next=kvn,
                q_prev=[blk[b][r] for b in range(bs)], q_next=[blk[b][n - r - 1] for b in range(bs)])


def test_token_walk_agrees_with_the_page_formulas():
    """The simulated shard/all-gather reproduces every list the page's
    formulas give, over random uneven, multi-sequence, prefixed batches, and
    satisfies the page's own consistency checks."""
    rng = random.Random(11)
    for cp in (2, 3, 4, 5, 8):
        for _ in range(12):
            bs, lens = _random_batch(rng, cp)
            prefix = [rng.choice([0, 0, 3, 29]) for _ in range(bs)]
            seq = [p + e for p, e in zip(prefix, lens)]
            for r in range(cp):
                m = zigzag_meta.build(cp, r, sum(lens), seq_lens=seq, extend_lens=lens)
                for key, want in _page_formulas(cp, r, lens, prefix).items():
                    assert getattr(m, key) == want, (cp, r, lens, key)
                # the page's consistency checks
                n = 2 * cp
                assert len(m.split_list) == bs * n and sum(m.split_list) == m.total_seq_lens
                assert len(m.zigzag_index) == 2 * bs and len(m.cp_reverse_index) == bs * n
                assert sorted(m.cp_reverse_index) == list(range(bs * n))
                assert sum(m.per_rank_actual_token) == m.total_seq_lens
                assert m.cu_seqlens_q_prev == [0] + list(itertools.accumulate(m.q_prev))
                assert m.cu_seqlens_q_next == [0] + list(itertools.accumulate(m.q_next))
