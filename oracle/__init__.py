"""CPU oracle for zigzag context-parallel prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or helpers with the HIP library in ``context_prefill_attention_amd``.

The oracle is written in plain Python integers (metadata and index maps) and
numpy float64 (attention), straight from the definitions on the source pages.
Citation keys used in this package:

[P1] "Zigzag cp #3" pull request page (alexsun07/sglang): AITER backend wired
     into prefill context parallelism on ROCm.
[P2] vllm-omni pull request #7937, "Compose Ulysses with AllGather-KV as a 2D
     SP topology": the local-Q / global-KV packed contract.
[P3] sglang pull request #39724, "Prefill context parallel E2E support".
[P4] prhub report on sglang pull request #34485 (AITer backend accepts
     grouped-query K/V): the GQA/MQA head-ratio contract and 1/sqrt(D) scale.
[P5] sglang source page ``python/sglang/srt/layers/cp/zigzag.py``: module
     docstring (block layout), ``ZigzagContextParallelMetadata``,
     ``ZigzagCPStrategy.can_apply``, ``build_metadata``, ``shard_*``,
     ``gather_*``, ``run_attention``, ``materialize_full_kv`` and
     ``_all_gather_reorganized``.

Modules:
  zigzag_meta  -- metadata lists of [P5] build_metadata (pure Python ints)
  layout       -- shard, all-gather buffer, rerange and KV-pool scatter as
                  index maps (numpy, bit copies)
  attention    -- fp64 softmax attention per segment, the zigzag rank share
                  and the AllGather-KV local-Q/global-KV variant

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
pages or mathematics fix (printed layouts, closed forms, brute force on tiny
inputs, a library special case); none is "parity unpinned".
"""

from . import zigzag_meta, layout, attention  # noqa: F401

__all__ = ["zigzag_meta", "layout", "attention"]
