"""Oracle for exact attention forward over packed variable-length sequences.

TEST INFRASTRUCTURE.  A plain, slow, float64 CPU implementation written from
the FlashAttention pages.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library and its
Python binding never import, call or link anything here, and nothing here
imports them: the two sides share only the seeded inputs of ``fa_synth``.

Contents
  * :mod:`oracle.cu_seqlens`     -- lengths and row offsets from cumulative offsets
  * :mod:`oracle.tile_map`       -- the flat (sequence, q-block) work-item map
  * :mod:`oracle.attention`      -- materialised fp64 attention (the definition)
  * :mod:`oracle.attention_grad` -- its gradients dq, dk, dv (chain rule on the
    materialised matrices)
  * :mod:`oracle.kvcache`        -- attention against a (paged) key/value cache
    with per-sequence lengths and left padding (the decode-shaped case)
  * :mod:`oracle.online_softmax` -- fp64 tile-by-tile emulation of the online
    softmax, used only to pin the claim that rescaled running statistics give
    the global softmax

Every function is pinned by ``tests/test_oracle_*.py`` against values printed
on the pages, closed forms, invariants, brute force and a library routine.
"""
from .cu_seqlens import lengths_from_cu, check_cu_seqlens, row_offset
from .tile_map import tile_map, tile_items
from .attention import attention_fwd, attention_rows, visible_mask, flops_visible_pairs, kv_head_of
from .attention_grad import attention_bwd, attention_loss
from .kvcache import attention_kvcache, cache_positions, gather_cache
from .online_softmax import online_softmax_attention, blockwise_normalised_attention

__all__ = [
    "lengths_from_cu",
    "check_cu_seqlens",
    "row_offset",
    "tile_map",
    "tile_items",
    "attention_fwd",
    "attention_rows",
    "visible_mask",
    "flops_visible_pairs",
    "kv_head_of",
    "attention_bwd",
    "attention_loss",
    "attention_kvcache",
    "cache_positions",
    "gather_cache",
    "online_softmax_attention",
    "blockwise_normalised_attention",
]
