"""Attention with per-head sink logits on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of ``libattnsink.so``
(``include/attn_sink.h``); this package is its thin Python binding. Using any binding
name requires the built library (``python -m gqa_attention_sinks_sink_amd.build``); a
missing library raises ImportError, there is no fallback.
"""
import importlib

__version__ = "0.1.0"

_BINDING_NAMES = (
    "AttnSinkError", "EXPORTED_SYMBOLS", "attn_sink_decode_paged", "attn_sink_decode_paged_partials",
    "attn_sink_prefill_paged", "attn_sink_decode_paged_tree", "attn_sink_rope_append",
    "attn_sink_decode_workspace_size",
    "attn_sink_merge_partials", "attn_sink_prefill", "attn_sink_status_string", "attn_sink_version",
    "attn_sink_decode_workspace_layout", "decode_workspace_layout", "attn_sink_decode_paged_noalloc",
    "attn_sink_decode_noalloc_capacity", "attn_sink_decode_paged_tree_partials",
    "attn_sink_decode_paged_range_partials", "attn_sink_decode_plan_chunk", "lib",
)
__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    # The binding loads the shared library on first use, so that the build module can run
    # before the library exists.
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module("._lib", __name__), name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
