"""Plain float64 CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  No torch, no code
shared with the HIP library.

Array conventions (all numpy):

* caches ``k_cache`` / ``v_cache``: ``[num_blocks, kv_heads, block_size, head_dim]``
  for one layer; element type float32, or uint16 holding bfloat16 bit patterns;
* ``block_tables``: int ``[num_seqs, max_blocks_per_seq]``, physical block ids in
  logical order;
* ``seq_lens``: int ``[num_seqs]``, number of cached positions each query sees;
* ``q``: ``[num_seqs, num_heads, head_dim]`` (same element type as the caches).

Decode results are float64.  Append and block copy work on the raw element
bits, so they are exact for either element type.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Capacity arithmetic and address translation
# --------------------------------------------------------------------------

def block_layout(tokens: int, block_size: int) -> tuple[int, int]:
    """Blocks one unshared sequence occupies, and its unused tail slots.

    lihaoran.work PagedAttention explainer, section "How many tail slots
    remain unused?": the block count is the ceiling of tokens / block_size
    (computed here as a negated floor division of the negated count), and
    the unused slots are the capacity of those blocks minus the tokens, a
    number in [0, block_size - 1] for a non-empty sequence and 0 for an
    empty one.  Negative token counts and non-positive block sizes raise
    ValueError (the page's helper rejects them the same way).
    """
    if tokens < 0 or block_size <= 0:
        raise ValueError(f"block_layout: bad sizes tokens={tokens} block_size={block_size}")
    blocks = -(-tokens // block_size)
    return blocks, blocks * block_size - tokens


def translate(table_row, position: int, block_size: int) -> tuple[int, int]:
    """Physical (block, slot) that holds cached position ``position``.

    lihaoran.work PagedAttention explainer, section "A block table maps
    logical order to physical storage": the logical block of zero-based
    position t is t // b, the slot inside it is t % b, and the table entry
    for that logical block names the physical block.
    """
    logical = position // block_size
    slot = position - logical * block_size
    return int(table_row[logical]), int(slot)


# --------------------------------------------------------------------------
# Element decoding
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64.

    A bfloat16 is the upper 16 bits of an IEEE-754 binary32, so widening the
    pattern to 32 bits with 16 zero bits below gives the same number.
    """
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    """float32 arrays as float64; uint16 arrays read as bfloat16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"oracle: unsupported element type {x.dtype}")


# --------------------------------------------------------------------------
# Gather through the block table
# --------------------------------------------------------------------------

def gather_history(k_cache, v_cache, table_row, seq_len: int, block_size: int):
    """Logical K and V history of one sequence, assembled block by block.

    lihaoran.work explainer, section "A block table maps logical order to
    physical storage": entry j of a sequence's table names the physical block
    that holds logical block j, i.e. positions [j*b, (j+1)*b).  Taking the
    first ceil(seq_len / b) entries in order, laying each named block's slots
    end to end, and keeping the first seq_len of them rebuilds the history in
    position order; the unused tail slots of the last block are dropped.
    Returns float64 arrays ``[seq_len, kv_heads, head_dim]`` (all KV heads).
    """
    _, kv_heads, _, head_dim = k_cache.shape
    blocks, _ = block_layout(seq_len, block_size)
    if blocks == 0:
        empty = np.empty((0, kv_heads, head_dim), dtype=np.float64)
        return empty, empty.copy()
    ids = [int(table_row[j]) for j in range(blocks)]
    # a block is [kv_heads, block_size, head_dim]: put its slots first
    keys = np.concatenate([to_f64(k_cache[p]).transpose(1, 0, 2) for p in ids], axis=0)
    values = np.concatenate([to_f64(v_cache[p]).transpose(1, 0, 2) for p in ids], axis=0)
    return keys[:seq_len], values[:seq_len]


def gather_history_vectorised(k_cache, v_cache, table_row, seq_len: int, block_size: int):
    """Same result as :func:`gather_history`, with numpy fancy indexing of
    every position's (block, slot) at once.

    Used for the large synthetic batches; a test checks both gathers against
    an independent position-by-position lookup.
    """
    positions = np.arange(seq_len, dtype=np.int64)
    blocks = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    slots = positions % block_size
    keys = to_f64(k_cache[blocks, :, slots, :])
    values = to_f64(v_cache[blocks, :, slots, :])
    return keys, values


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def attend(q_heads, keys, values, scale: float) -> np.ndarray:
    """Scaled dot-product attention of one decode query over its history.

    ``q_heads`` ``[num_heads, head_dim]``; ``keys``/``values``
    ``[seq_len, kv_heads, head_dim]``, all float64.

    The zenaique.com lookup code ends in ordinary scaled dot-product
    attention over the gathered keys and values, and the lihaoran.work
    explainer (section "A block table maps logical order to physical
    storage") states that attention still spans the whole visible history,
    so every one of the seq_len positions takes part.  Grouped-query
    attention: with G = num_heads / kv_heads, query head h reads KV head
    h // G (consecutive query heads share a KV head).  The softmax subtracts
    the row maximum before exponentiating, which leaves the result unchanged
    and keeps exp() finite.  An empty history gives a zero output.
    """
    num_heads, head_dim = q_heads.shape
    seq_len, kv_heads, _ = keys.shape
    if num_heads % kv_heads != 0:
        raise ValueError("num_heads must be a multiple of kv_heads")
    group = num_heads // kv_heads
    out = np.zeros((num_heads, head_dim), dtype=np.float64)
    if seq_len == 0:
        return out
    for head in range(num_heads):
        kv_head = head // group
        scores = scale * (keys[:, kv_head, :] @ q_heads[head])
        weights = np.exp(scores - scores.max())
        weights = weights / weights.sum()
        out[head] = weights @ values[:, kv_head, :]
    return out


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float, block_size: int,
                 seqs=None, literal: bool = False) -> np.ndarray:
    """Decode attention for every sequence (or the listed ``seqs``).

    For each sequence: gather its history through its block table, then
    :func:`attend`.  ``literal=True`` uses the block-by-block gather, else the
    fancy-index one.  Returns float64 ``[len(seqs), num_heads, head_dim]``.
    """
    q = np.asarray(q)
    if seqs is None:
        seqs = range(q.shape[0])
    seqs = list(seqs)
    gather = gather_history if literal else gather_history_vectorised
    out = np.empty((len(seqs), q.shape[1], q.shape[2]), dtype=np.float64)
    for i, s in enumerate(seqs):
        keys, values = gather(k_cache, v_cache, block_tables[s], int(seq_lens[s]), block_size)
        out[i] = attend(to_f64(q[s]), keys, values, scale)
    return out


def contiguous_decode(q, keys_per_seq, values_per_seq, scale: float) -> np.ndarray:
    """Decode attention over histories stored contiguously (no paging).

    The unpaged baseline the paged kernel must reproduce: the lihaoran.work
    explainer notes paging changes where the data lives, not what attention
    computes.  ``keys_per_seq[s]`` is ``[seq_len_s, kv_heads, head_dim]``.
    """
    q = np.asarray(q)
    out = np.empty(q.shape, dtype=np.float64)
    for s in range(q.shape[0]):
        out[s] = attend(to_f64(q[s]), to_f64(keys_per_seq[s]), to_f64(values_per_seq[s]), scale)
    return out


# --------------------------------------------------------------------------
# Layered pool: every layer's K and V in one block
# --------------------------------------------------------------------------

def layer_views(kv_pool, layer: int):
    """The per-layer K and V caches ``[num_blocks, kv_heads, block_size,
    head_dim]`` inside a layered pool ``[num_blocks, 2, num_layers, kv_heads,
    block_size, head_dim]`` (zenaique.com code box "Conceptual:
    PagedAttention block lookup": index 0 of the second axis holds K, 1 holds
    V).  numpy views: writes go to the pool."""
    return kv_pool[:, 0, layer], kv_pool[:, 1, layer]


def paged_decode_layered(q_layers, kv_pool, block_tables, seq_lens, scale: float,
                         block_size: int, layers=None, seqs=None) -> np.ndarray:
    """Decode attention of several layers over one layered pool.

    ``q_layers`` ``[num_layers, num_seqs, num_heads, head_dim]``.  Layout of
    the zenaique.com code box "Conceptual: PagedAttention block lookup": a
    physical block holds, for its block_size positions, K (index 0 of the
    second axis) and V (index 1) of every layer and KV head.  One table per
    sequence serves all layers: the history is rebuilt block by block as in
    :func:`gather_history`, each named block contributing all layers at once,
    and each layer then runs :func:`attend`.  Returns float64
    ``[len(layers), len(seqs), num_heads, head_dim]``.
    """
    q_layers = np.asarray(q_layers)
    num_layers = kv_pool.shape[2]
    layers = list(range(num_layers)) if layers is None else list(layers)
    seqs = list(range(q_layers.shape[1])) if seqs is None else list(seqs)
    out = np.empty((len(layers), len(seqs), q_layers.shape[2], q_layers.shape[3]), dtype=np.float64)
    for j, s in enumerate(seqs):
        seq_len = int(seq_lens[s])
        blocks, _ = block_layout(seq_len, block_size)
        ids = [int(block_tables[s][i]) for i in range(blocks)]
        # kv_pool[p, 0] is [layers, kv_heads, block_size, head_dim]: slots first
        parts_k = [to_f64(kv_pool[p, 0]).transpose(2, 0, 1, 3) for p in ids]
        parts_v = [to_f64(kv_pool[p, 1]).transpose(2, 0, 1, 3) for p in ids]
        shape = (0, num_layers) + kv_pool.shape[3:4] + kv_pool.shape[5:6]
        keys = np.concatenate(parts_k, axis=0)[:seq_len] if ids else np.empty(shape)
        values = np.concatenate(parts_v, axis=0)[:seq_len] if ids else np.empty(shape)
        for i, layer in enumerate(layers):
            out[i, j] = attend(to_f64(q_layers[layer, s]), keys[:, layer], values[:, layer], scale)
    return out


# --------------------------------------------------------------------------
# Prefill: a chunk of queries per sequence, causal
# --------------------------------------------------------------------------

def chunk_positions(seq_len: int, query_len: int) -> np.ndarray:
    """Positions of a sequence's prefill queries.

    The chunk's keys and values are already in the cache, so its queries are
    the last ``query_len`` of the ``seq_len`` cached positions: L - n, ...,
    L - 1 (a whole prompt when n = L; a later chunk after a cached prefix
    when n < L, the prefix-reuse case of "How PagedAttention works", section
    "A strong answer").
    """
    if query_len < 0 or query_len > seq_len:
        raise ValueError(f"chunk of {query_len} queries in a sequence of {seq_len}")
    return np.arange(seq_len - query_len, seq_len, dtype=np.int64)


def visible_prefix(position: int, seq_len: int) -> int:
    """How many positions the query at ``position`` attends: [0, position].

    lihaoran.work explainer, section "A block table maps logical order to
    physical storage": full causal attention covers the visible history, so
    a query sees itself and every earlier position, never a later one.
    """
    return position + 1


def paged_prefill(q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale: float,
                  block_size: int, rows=None, literal: bool = False) -> np.ndarray:
    """Causal attention of each sequence's chunk of queries over its paged history.

    ``q`` ``[num_queries, num_heads, head_dim]`` holds the sequences' chunks
    one after another: sequence s owns rows [start_s, start_s + query_lens[s])
    with start_s the sum of the earlier query_lens.  Its history is gathered
    through its block table as in decode; the query at position p
    (:func:`chunk_positions`) then attends the first :func:`visible_prefix`
    positions with :func:`attend`.  ``rows`` limits the work to the listed
    global query rows.  Returns float64 ``[len(rows), num_heads, head_dim]``.
    """
    q = np.asarray(q)
    query_lens = np.asarray(query_lens, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(query_lens)])
    if rows is None:
        rows = range(int(starts[-1]))
    rows = [int(r) for r in rows]
    gather = gather_history if literal else gather_history_vectorised
    histories = {}
    out = np.empty((len(rows), q.shape[1], q.shape[2]), dtype=np.float64)
    for i, r in enumerate(rows):
        s = int(np.searchsorted(starts, r, side="right")) - 1
        seq_len = int(seq_lens[s])
        if s not in histories:
            histories[s] = gather(k_cache, v_cache, block_tables[s], seq_len, block_size)
        keys, values = histories[s]
        position = int(chunk_positions(seq_len, int(query_lens[s]))[r - int(starts[s])])
        seen = visible_prefix(position, seq_len)
        out[i] = attend(to_f64(q[r]), keys[:seen], values[:seen], scale)
    return out


# --------------------------------------------------------------------------
# Cache writes
# --------------------------------------------------------------------------

def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, block_size: int) -> None:
    """Write new tokens' keys and values into their cache slots, in place.

    "How PagedAttention works", section "A strong answer": each decode step
    adds one token to a sequence's cache.  A slot number s names physical
    block s // b, position s % b inside it (the same block/offset split as
    the block table translation); a negative slot is padding and is skipped.
    Works on raw element bits, so the copy is exact.
    """
    for token, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        k_cache[block, :, offset, :] = k_new[token]
        v_cache[block, :, offset, :] = v_new[token]


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """Copy-on-write block copy, in place.

    "How PagedAttention works", feature table row on beam search / parallel
    sampling, and the zenaique.com follow-up on beam search: when a shared
    block is about to diverge, a fresh block receives a full copy of it.
    Each (src, dst) pair copies every KV head and every slot of block src,
    keys and values, into block dst.  Destinations never overlap sources.
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs) -> None:
    """Move whole blocks from one pool into another, in place.

    "How PagedAttention works", feature table row on preemption and section
    "What interviewers probe next": a preempted sequence's blocks go to pinned
    host memory (and come back) a block at a time.  Each (src, dst) pair
    copies every KV head and every slot of block src of the source pool,
    keys and values, into block dst of the destination pool; the two pools
    share the block shape and may differ in size.  Raw bits, so exact.
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]
