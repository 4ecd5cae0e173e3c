"""CPU fp64 oracle for attention with per-head sink logits.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only the test-suite, the smoke check in ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
kernels or their C ABI, and it never reads a value produced by them.

What it computes (source: "GPT-OSS on Day 0", section "Attention sinks"): each
attention head carries a learned sink logit that enters the softmax next to the
scaled Q.K scores; the sink has no value vector. ``attention.attend`` writes out that
definition directly (one softmax over [scores, sink]). ``attention.online_partials``
follows the streaming form the same section describes (running max seeded with the
head's sink, scale initialised to 1, sink only in the first KV chunk) and
``attention.merge`` combines split-KV partials by log-sum-exp. ``rope`` holds the step
before attention for new tokens: YaRN rotary encoding (named by the same page) and the
write of the new K/V into the paged cache.

Every function is pinned by tests under ``tests/`` that do not go through the
oracle's own formulas (library attention with the sink disabled, closed forms,
invariants, brute force at 50 digits, hand-derived fixtures under ``tests/golden``).
The only convention the pages leave open that changes a result is whether the
returned log-sum-exp includes the sink term; here it does (parity unpinned by the
pages: a stated reading).
"""
from .attention import (  # noqa: F401
    attend, attention_weights, prefill_varlen, gather_pages, decode_paged, prefill_paged,
    tree_visible, decode_paged_tree,
    online_partials, split_decode, merge, plan_chunks,
)
from .rope import yarn_frequencies, rotate, rope_append  # noqa: F401
