"""CPU oracle for paged decode (and chunked prefill) attention. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
product path (``paged_kv_cache_163_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.

Everything here is plain numpy in float64, written to be checked by eye
against the pages it cites, not to be fast.  Each function names the page and
section whose statement it follows.  The pages are:

* "How PagedAttention works" (aiinfrainterviews.com), sections
  "TL;DR" and "A strong answer";
* "What KV cache problem does paged attention in vLLM solve, and which
  operating system idea does it use?" (zenaique.com), the conceptual
  block-lookup code box, the comparison table and the follow-up question on
  beam search;
* the lihaoran.work PagedAttention explainer, sections "A block table maps
  logical order to physical storage", "How many tail slots remain unused?"
  and "Shared prefixes need matching computation".

Parity status: every function is pinned by ``tests/test_oracle.py`` (values
printed on the pages, closed forms, brute force and invariants).  None is
"parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    attend,
    bf16_bits_to_f64,
    block_layout,
    chunk_positions,
    contiguous_decode,
    copy_blocks,
    gather_history,
    gather_history_vectorised,
    kv_append,
    layer_views,
    paged_decode,
    paged_decode_layered,
    paged_prefill,
    swap_blocks,
    to_f64,
    translate,
    visible_prefix,
)
