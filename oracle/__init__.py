"""CPU oracle for the causal KV-cache attention hot path of Ca2-VDM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call, link or
execute anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` do. The oracle shares no code with
the HIP library: no kernels, headers, helpers, tables or pre-/post-processing.
The only shared module is ``synth`` (seeded random draws), which holds none of
the method's arithmetic.

Everything here is the plain definition, written in float64 with
max-subtracted softmax and no streaming, blocking or fusion. Each function
cites the passage of the source pages it follows. The pages are:

* "Ca2-VDM notes" -- papernotes.org, "Ca2-VDM: Efficient Autoregressive Video
  Diffusion Model with Causal Generation and Cache Sharing" (ICML 2025 notes);
  sections are named by their headings (整体框架 overall framework, 关键设计
  key designs 1-5, 损失函数/训练策略 training, the speed and memory tables).
* "Ca2-VDM abstract page" -- bohrium.dp.tech, arXiv 2411.16375 abstract and
  its "Formula Representation" section.
* "Ca2-VDM summary" -- atlas.scime.ai summary (Approach, Key results).

Pin status of each function is stated in its docstring and collected in the
design notes. Where the pages leave a step open, the reading taken is named
in the docstring, and the function is pinned for that reading by a closed
form or a construction other than its own.
"""
from .attention import (
    softmax_rows,
    temporal_attn_ref,
    spatial_attn_ref,
    spatial_attn_selfrepeat_ref,
    masked_causal_attn_ref,
    full_recompute_temporal_ref,
    bidirectional_temporal_ref,
)
from .cache import (
    TemporalQueue,
    SpatialCache,
    tpe_index_ref,
    bytes_resident_ref,
)
from .projection import qkv_proj_ref, qkv_proj_tpe_ref
from .rollout import ar_schedule, RolloutOracle

__all__ = [
    "softmax_rows", "temporal_attn_ref", "spatial_attn_ref",
    "spatial_attn_selfrepeat_ref", "masked_causal_attn_ref",
    "full_recompute_temporal_ref", "bidirectional_temporal_ref", "TemporalQueue", "SpatialCache",
    "tpe_index_ref", "bytes_resident_ref", "qkv_proj_ref", "qkv_proj_tpe_ref", "ar_schedule",
    "RolloutOracle",
]
