"""The whole device step (KV scatter, rerange of K and V, one tensor at a
time or both in one launch, fused attention)
captured in a HIP graph and replayed.

The entry points allocate nothing, never synchronise and launch on the
caller's stream, so one batch's step can be captured once and replayed.
Between replays the outputs are overwritten with NaN by eager work; every
replay must reproduce the eager results bit for bit (the kernels are
deterministic)."""

import math

import numpy as np
import pytest
import torch

import context_prefill_attention_amd as cpa
import synth
from oracle import layout, zigzag_meta

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("paired", [False, True], ids=["rerange_each", "rerange_kv"])
def test_step_captured_in_a_graph_replays_bit_exact(paired):
    cp, rank, lens, h_q, h_kv, d, ps = 4, 1, [300, 128, 77], 16, 2, 128, 16
    total = sum(lens)
    qg, kg, vg = synth.normal_bf16(71, (total, h_q, d), (total, h_kv, d), (total, h_kv, d))
    mo = zigzag_meta.build(cp, rank, total, extend_lens=lens)
    bits = lambda t: t.view(torch.int16).numpy()
    k_gath = torch.from_numpy(layout.gathered_buffer(bits(kg), mo)).view(torch.bfloat16).cuda()
    v_gath = torch.from_numpy(layout.gathered_buffer(bits(vg), mo)).view(torch.bfloat16).cuda()
    q_loc = torch.from_numpy(layout.shard(bits(qg), mo)).view(torch.bfloat16).cuda()
    w = synth.Workload(name="graph", seed=71, causal=True, h_q=h_q, h_kv=h_kv, d=d, page_size=ps,
                       contiguous_kv=False, cp_size=cp)
    indptr, indices, npages = synth.page_table(w, lens)
    ip, ix = torch.from_numpy(indptr).cuda(), torch.from_numpy(indices).cuda()
    meta = cpa.meta_build(cp, rank, lens, attn_group=h_q // h_kv, device="cuda")
    kp = torch.zeros(npages, ps, h_kv, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    k_orig = torch.empty(total, h_kv, d, dtype=torch.bfloat16, device="cuda")
    v_orig = torch.empty_like(k_orig)
    out = torch.empty_like(q_loc)
    scale = 1 / math.sqrt(d)

    def step():
        cpa.kv_scatter(meta, k_gath, v_gath, kp, vp, ps, ip, ix)
        if paired:
            cpa.zigzag_rerange_kv(meta, k_gath, k_orig, v_gath, v_orig, cpa.GATHERED_TO_ORIG)
        else:
            cpa.zigzag_rerange(meta, k_gath, k_orig, cpa.GATHERED_TO_ORIG)
            cpa.zigzag_rerange(meta, v_gath, v_orig, cpa.GATHERED_TO_ORIG)
        cpa.prefill_attn(q_loc, kp, vp, out, meta, scale, ps, ip, ix)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (kp, vp, k_orig, v_orig, out)]
    assert torch.isfinite(out).all()
    assert torch.equal(k_orig.view(torch.int16).cpu(), kg.view(torch.int16))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (kp, vp, k_orig, v_orig, out):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("k_pool", "v_pool", "k_orig", "v_orig", "out"), (kp, vp, k_orig, v_orig, out), ref):
            # the pool slots of no token are not written by the step: they keep the NaN fill
            if name in ("k_pool", "v_pool"):
                rows = np.zeros(npages * ps, dtype=bool)
                for b in range(len(lens)):
                    first = int(indptr[b])
                    for tkn in range(lens[b]):
                        rows[int(indices[first + tkn // ps]) * ps + tkn % ps] = True
                sel = torch.from_numpy(rows).cuda()
                tv, rv = t.view(-1, h_kv, d)[sel], r.view(-1, h_kv, d)[sel]
            else:
                tv, rv = t, r
            assert torch.equal(tv.view(torch.int16), rv.view(torch.int16)), f"replay {rep}: {name}"
