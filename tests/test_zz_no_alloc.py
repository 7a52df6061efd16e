"""cp_prefill_attn_noalloc, the attention entry point for callers that cannot
allocate: its run-time job counters live in the library's per-device array
instead of the metadata blob.  Two calls in a row through the C ABI, the
second on a smaller input, each checked bit for bit against cp_prefill_attn
on the same inputs (the same kernel; a job's result does not depend on where
it runs), every row written, and the blob left as it was."""

import math

import pytest
import torch

import context_prefill_attention_amd as cpa
import synth

pytestmark = pytest.mark.gpu

ROWS_PER_ITEM = 256


def _case(n_jobs, h_kv, seed, h_q=32, d=128, kv_len=3072, ps=64):
    """AllGather-KV slice with exactly n_jobs jobs of kv_len / 64 key tiles
    (at least 48 on average and more jobs than CUs: the counters are used)."""
    group = h_q // h_kv
    q_total = n_jobs // h_kv * (ROWS_PER_ITEM // group)
    npages = -(-kv_len // ps)
    qg, kg, vg = synth.normal_bf16(seed, (q_total, h_q, d), (npages * ps, h_kv, d), (npages * ps, h_kv, d))
    meta = cpa.allgather_meta_build(q_total, q_total, kv_len, group, device="cuda")
    assert meta.n_work * h_kv == n_jobs and meta.mean_item_tiles >= 48
    pool = lambda t: t.view(npages, ps, h_kv, d).cuda()
    indptr = torch.tensor([0, npages], dtype=torch.int32, device="cuda")
    indices = torch.arange(npages, dtype=torch.int32, device="cuda")
    return dict(q=qg.cuda(), kp=pool(kg), vp=pool(vg), meta=meta, ps=ps, ip=indptr, ix=indices,
                scale=1 / math.sqrt(d))


def _run(c, noalloc):
    out = torch.full(c["q"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    cpa.prefill_attn(c["q"], c["kp"], c["vp"], out, c["meta"], c["scale"], c["ps"], c["ip"], c["ix"],
                     noalloc=noalloc)
    return out


def test_noalloc_two_calls_match_prefill_attn():
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    big = _case(-(-(3 * n_cu + 40) // 8) * 8, 8, 41)
    small = _case(n_cu + 3, 1, 42)                       # the second call's input is smaller
    blobs = [c["meta"].d_blob.clone() for c in (big, small)]
    got = []
    for name, c in (("big", big), ("small", small)):      # two no-alloc calls in a row
        print("noalloc call", name, flush=True)
        got.append(_run(c, True))
    torch.cuda.synchronize()
    for (name, c), g, b in zip((("big", big), ("small", small)), got, blobs):
        assert torch.isfinite(g).all(), f"{name}: rows left unwritten"
        assert torch.equal(c["meta"].d_blob, b), f"{name}: the blob was written"
        ref = _run(c, False)
        torch.cuda.synchronize()
        assert torch.equal(g.view(torch.int16), ref.view(torch.int16)), f"{name}: differs from cp_prefill_attn"
