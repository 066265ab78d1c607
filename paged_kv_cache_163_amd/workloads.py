"""Seeded synthetic decode batches shaped like the pages' workloads.

This module feeds both the HIP path and the CPU oracle.  It holds no attention
arithmetic and no position-to-slot gather: it plays the block manager only
(drawing sequence lengths, handing out physical blocks from a seeded free
list, reference counting shared blocks, choosing the slot a new token goes
to) and fills physical blocks with random values.  Numpy only, no torch.

Element encoding on the host: float32 arrays for "f32"; uint16 arrays holding
bfloat16 bit patterns (round-to-nearest-even from float32 N(0,1) draws) for
"bf16".  Every slot that holds no live token (tail slots of a sequence's last
block, free blocks, the padding block that table entries past a sequence's
last block point at) is filled with NaN, so any read of dead data shows up.

Workloads (all use ``numpy.random.default_rng(seed)``, seed 0 by default):

* ``tiny``: 4 sequences of lengths 10, 1, 16, 37, block size 4, 8 query /
  2 KV heads, head_dim 64, float32, pool of 32 blocks; sequence 0's table is
  [5, 1, 7] (the worked example of the lihaoran.work explainer).
* ``llama70b``: one Llama-3.1-70B-shaped layer (64 query / 8 KV heads,
  head_dim 128), bfloat16, block size 16, 256 chat sequences with context
  U{500..700} + U{0..250} tokens, blocks drawn from a pool of 20,000.
* ``shared_prefix``: 200 sequences sharing one 2,000-token prefix (125 blocks
  of 16, refcount 200) plus private tails of U{1..400} tokens; then 16 beams
  fork from one sequence whose last block is partly filled, each beam gets a
  copy-on-write copy of that block and writes its own next token into it.
* ``long_context``: 16 sequences of 8,192 tokens (512 blocks each) scattered
  in a 10,000-block pool.
* ``sweep``: 512 sequences, lengths log-uniform in [16, 4096], 32 query /
  8 KV heads, block size in {16, 32, 64}, head_dim in {64, 128}.
* ``llama70b_contiguous``: the llama70b batch (same lengths, queries, new
  tokens and cache contents) with physically sequential blocks: sequence s
  holds consecutive block ids right after sequence s - 1.  Decode over it
  reads the same logical K/V, so its outputs equal llama70b's; timing the
  two measures what the random placement of the table costs.

Every builder takes ``fill``: with ``fill=False`` the caches are left
unwritten (``numpy.empty``), for callers that only need the tables, lengths
and slots and fill device pools themselves (timing runs).

Configurations with a decode step (tiny, llama70b, shared_prefix, sweep)
describe the cache *before* the step; the step writes one new token per
appending sequence at position ``pre_len`` (via ``slot_mapping``) and the
decode then attends over ``seq_lens`` (= ``pre_len + 1`` for those sequences).
The block table already lists the block that position falls in.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# element helpers
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.

    NaN inputs map to the canonical quiet NaN 0x7FC0."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    nan = np.isnan(x)
    u = x.view(np.uint32)
    bump = u >> np.uint32(16)
    bump &= np.uint32(1)
    bump += np.uint32(0x7FFF)
    u += bump
    u >>= np.uint32(16)
    out = u.astype(np.uint16)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    vals = rng.standard_normal(shape, dtype=np.float32)
    if dtype != "bf16":
        return vals
    u = vals.view(np.uint32)               # N(0,1) draws are never NaN
    bump = u >> np.uint32(16)
    bump &= np.uint32(1)
    bump += np.uint32(0x7FFF)
    u += bump
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def _stream(seed: int, kind: int, index: int) -> np.random.Generator:
    """Independent generator for one sequence's cache contents, so that the
    blocks can be filled in parallel with the same result for any thread count."""
    return np.random.default_rng([int(seed), int(kind), int(index)])


_FILL_THREADS = max(1, min(8, os.cpu_count() or 1))


def _nan_pool(shape, dtype: str, fill: bool = True) -> np.ndarray:
    if not fill:
        return np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if dtype == "bf16":
        return np.full(shape, BF16_NAN, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# --------------------------------------------------------------------------
# block manager (allocation + refcounts)
# --------------------------------------------------------------------------

class BlockPool:
    """Free list of physical block ids in a seeded random order, with refcounts.

    "How PagedAttention works" (section "A strong answer"): blocks are handed
    out on demand, a shared prefix is one set of blocks with a refcount per
    block, and a fork copies only the block that diverges.
    """

    def __init__(self, num_blocks: int, order: np.ndarray):
        self.num_blocks = int(num_blocks)
        self._free = [int(b) for b in order]
        self._next = 0
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)

    def take(self, n: int = 1) -> list[int]:
        if self._next + n > len(self._free):
            raise MemoryError(f"block pool exhausted: want {n}, "
                              f"{len(self._free) - self._next} free")
        ids = self._free[self._next:self._next + n]
        self._next += n
        for b in ids:
            self.refcount[b] += 1
        return ids

    def share(self, ids) -> None:
        for b in ids:
            self.refcount[b] += 1

    @property
    def used(self) -> int:
        return int((self.refcount > 0).sum())


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------

@dataclass
class DecodeWorkload:
    name: str
    dtype: str                      # "f32" or "bf16"
    num_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: np.ndarray                   # [B, Hq, D]
    k_cache: np.ndarray             # [NB, Hkv, b, D]  state before the step
    v_cache: np.ndarray
    block_tables: np.ndarray        # int32 [B, max_blocks_per_seq]
    seq_lens: np.ndarray            # int32 [B]  lengths the decode attends over
    pre_lens: np.ndarray            # int32 [B]  cached lengths before the step
    k_new: np.ndarray               # [T, Hkv, D] tokens written by the step
    v_new: np.ndarray
    slot_mapping: np.ndarray        # int64 [T]   destination slot per new token
    append_seq: np.ndarray          # int64 [T]   sequence each new token belongs to
    cow_pairs: np.ndarray           # int64 [n, 2] (src, dst) block copies of the step
    padding_block: int
    refcount: np.ndarray            # int64 [NB]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def per_sequence_append(w: "DecodeWorkload"):
    """The step's new tokens laid out one row per sequence, for the fused
    append+decode call: (k_new [B, Hkv, D], v_new, slot_mapping int64 [B]),
    zero rows and slot -1 for sequences that append nothing."""
    B = w.num_seqs
    k = np.zeros((B,) + w.k_new.shape[1:], dtype=w.k_new.dtype)
    v = np.zeros_like(k)
    slots = np.full(B, -1, dtype=np.int64)
    k[w.append_seq] = w.k_new
    v[w.append_seq] = w.v_new
    slots[w.append_seq] = w.slot_mapping
    return k, v, slots


def kv_bytes_per_token(kv_heads: int, head_dim: int, elem_bytes: int, layers: int = 1) -> int:
    """Bytes of K plus V that one token occupies (per layer unless ``layers``)."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def decode_kv_bytes(seq_lens, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Live K/V bytes one decode pass must read: live tokens only, no tail slots."""
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * kv_bytes_per_token(
        kv_heads, head_dim, elem_bytes)


# --------------------------------------------------------------------------
# generic builder
# --------------------------------------------------------------------------

def unique_kv_bytes(block_tables, seq_lens, block_size: int, kv_heads: int, head_dim: int,
                    elem_bytes: int) -> int:
    """K+V bytes of the distinct live (physical block, slot) positions the
    tables reach: a block shared by several tables counts once, filled as far
    as its fullest reader."""
    fill: dict[int, int] = {}
    for s, n in enumerate(np.asarray(seq_lens)):
        n = int(n)
        for j in range(_ceil_div(n, block_size)):
            b = int(block_tables[s, j])
            fill[b] = max(fill.get(b, 0), min(block_size, n - j * block_size))
    return int(sum(fill.values())) * 2 * kv_heads * head_dim * elem_bytes


def _fill_sequence(rng, k_cache, v_cache, blocks, live_tokens: int, dtype: str):
    """Random K/V in the first ``live_tokens`` slots of ``blocks`` (in order),
    NaN in the remaining slots of the last block."""
    nb = len(blocks)
    if nb == 0:
        return
    _, kv_heads, bs, head_dim = k_cache.shape
    idx = np.asarray(blocks, dtype=np.int64)
    k_cache[idx] = _draw(rng, (nb, kv_heads, bs, head_dim), dtype)
    v_cache[idx] = _draw(rng, (nb, kv_heads, bs, head_dim), dtype)
    filled_in_last = live_tokens - (nb - 1) * bs
    if filled_in_last < bs:
        nan = _nan_pool((kv_heads, bs - filled_in_last, head_dim), dtype)
        k_cache[idx[-1], :, filled_in_last:, :] = nan
        v_cache[idx[-1], :, filled_in_last:, :] = nan


def _fill_all(seed: int, kind: int, k_cache, v_cache, block_lists, live_counts, dtype: str):
    """Fill each sequence's private blocks from its own stream, in parallel
    (the block lists are disjoint, so the writes never overlap)."""
    def one(i):
        _fill_sequence(_stream(seed, kind, i), k_cache, v_cache, block_lists[i],
                       int(live_counts[i]), dtype)
    with ThreadPoolExecutor(_FILL_THREADS) as ex:
        list(ex.map(one, range(len(block_lists))))


def _append_slot(blocks: list[int], pre_len: int, bs: int, pool: BlockPool) -> int:
    """Slot the token at position ``pre_len`` goes to; takes a fresh block when
    the sequence's last block is full (or it has none)."""
    held = len(blocks)
    if pre_len == held * bs:              # no room left in the held blocks
        blocks.extend(pool.take(1))
        return blocks[-1] * bs
    fill = pre_len - (held - 1) * bs      # slots already used in the last block
    return blocks[-1] * bs + fill


def _pack_tables(tables: list[list[int]], padding: int) -> np.ndarray:
    width = max(1, max(len(t) for t in tables))
    out = np.full((len(tables), width), padding, dtype=np.int32)
    for s, t in enumerate(tables):
        out[s, :len(t)] = t
    return out


def build_private(name: str, pre_lens, *, dtype: str, num_heads: int, kv_heads: int,
                  head_dim: int, block_size: int, num_blocks: int, append: bool,
                  seed: int = 0, fixed_tables: dict | None = None, rng=None,
                  scale: float | None = None, meta: dict | None = None,
                  sequential: bool = False, fill: bool = True) -> DecodeWorkload:
    """Sequences with private blocks only.

    ``fixed_tables`` maps a sequence index to a block list it must use (and the
    allocator skips those ids).  Draw order on ``rng`` (default_rng(seed) unless
    the caller already drew lengths from it): placement permutation, q, new
    tokens.  Sequence s's cache contents come from its own stream
    default_rng([seed, 7, s]).  ``sequential`` hands blocks out in id order
    instead of the drawn permutation (which is still drawn, so q and the new
    tokens are the same either way).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    pre_lens = np.asarray(pre_lens, dtype=np.int64)
    nseq = len(pre_lens)
    bs = block_size
    fixed_tables = fixed_tables or {}
    reserved = {b for t in fixed_tables.values() for b in t}
    order = rng.permutation(num_blocks)
    if sequential:
        order = np.arange(num_blocks)
    order = np.asarray([b for b in order if b not in reserved], dtype=np.int64)
    pool = BlockPool(num_blocks, order)
    padding = pool.take(1)[0]
    tables: list[list[int]] = []
    for s in range(nseq):
        need = _ceil_div(int(pre_lens[s]), bs)
        if s in fixed_tables:
            t = list(fixed_tables[s])
            assert len(t) == need, "fixed table does not match the sequence length"
            pool.share(t)
        else:
            t = pool.take(need)
        tables.append(t)
    q = _draw(rng, (nseq, num_heads, head_dim), dtype)
    k_cache = _nan_pool((num_blocks, kv_heads, bs, head_dim), dtype, fill)
    v_cache = _nan_pool((num_blocks, kv_heads, bs, head_dim), dtype, fill)
    if fill:
        _fill_all(seed, 7, k_cache, v_cache, tables, pre_lens, dtype)
    if append:
        slots = np.asarray([_append_slot(tables[s], int(pre_lens[s]), bs, pool)
                            for s in range(nseq)], dtype=np.int64)
        k_new = _draw(rng, (nseq, kv_heads, head_dim), dtype)
        v_new = _draw(rng, (nseq, kv_heads, head_dim), dtype)
        seq_lens = pre_lens + 1
    else:
        slots = np.zeros((0,), dtype=np.int64)
        k_new = _draw(rng, (0, kv_heads, head_dim), dtype)
        v_new = _draw(rng, (0, kv_heads, head_dim), dtype)
        seq_lens = pre_lens.copy()
    return DecodeWorkload(
        name=name, dtype=dtype, num_heads=num_heads, kv_heads=kv_heads, head_dim=head_dim,
        block_size=bs, num_blocks=num_blocks,
        scale=float(scale if scale is not None else 1.0 / np.sqrt(head_dim)),
        q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=_pack_tables(tables, padding),
        seq_lens=seq_lens.astype(np.int32), pre_lens=pre_lens.astype(np.int32),
        k_new=k_new, v_new=v_new, slot_mapping=slots,
        append_seq=np.arange(slots.shape[0], dtype=np.int64),
        cow_pairs=np.zeros((0, 2), dtype=np.int64), padding_block=int(padding),
        refcount=pool.refcount.copy(), meta=dict(meta or {}))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def tiny(seed: int = 0, append: bool = True, fill: bool = True) -> DecodeWorkload:
    """4 sequences {10, 1, 16, 37}, b=4, 8/2 heads, D=64, fp32, 32-block pool.
    Sequence 0 uses table [5, 1, 7]."""
    return build_private(
        "tiny", [10, 1, 16, 37], dtype="f32", num_heads=8, kv_heads=2, head_dim=64,
        block_size=4, num_blocks=32, append=append, seed=seed,
        fixed_tables={0: [5, 1, 7]}, scale=1.0 / np.sqrt(64.0), fill=fill)


def llama70b(seed: int = 0, num_seqs: int = 256, append: bool = True,
             sequential: bool = False, fill: bool = True, tp: int = 1) -> DecodeWorkload:
    """One Llama-3.1-70B-shaped layer: 256 chat sequences, bf16, b=16, 20k blocks
    (``sequential``: the same batch on physically consecutive blocks; ``tp``:
    one GPU's share under tensor parallelism over ``tp`` GPUs, 8/tp KV heads
    and 64/tp query heads of every block, the same lengths and placement)."""
    if tp not in (1, 2, 4, 8):
        raise ValueError("tp must divide the 8 KV heads")
    rng = np.random.default_rng(seed)
    prompt = rng.integers(500, 700, size=num_seqs, endpoint=True)
    generated = rng.integers(0, 250, size=num_seqs, endpoint=True)
    name = "llama70b_contiguous" if sequential else "llama70b"
    if tp > 1:
        name += f"_tp{tp}"
    return build_private(
        name, prompt + generated, dtype="bf16",
        num_heads=64 // tp, kv_heads=8 // tp, head_dim=128, block_size=16, num_blocks=20000,
        append=append, rng=rng, seed=seed, sequential=sequential, fill=fill,
        meta={"prompt": "U{500..700}", "generated": "U{0..250}",
              "placement": "sequential" if sequential else "random", "tp": tp})


def llama70b_contiguous(seed: int = 0, fill: bool = True) -> DecodeWorkload:
    """The llama70b batch with each sequence's blocks physically consecutive."""
    return llama70b(seed=seed, sequential=True, fill=fill)


def llama70b_tp8(seed: int = 0, fill: bool = True) -> DecodeWorkload:
    """One GPU's share of the llama70b batch under 8-way tensor parallelism:
    one KV head and its 8 query heads of every block, the same lengths."""
    return llama70b(seed=seed, fill=fill, tp=8)


def long_context(seed: int = 0, fill: bool = True) -> DecodeWorkload:
    """16 sequences x 8,192 tokens (512 blocks each) in a 10,000-block pool."""
    return build_private(
        "long_context", [8192] * 16, dtype="bf16", num_heads=64, kv_heads=8, head_dim=128,
        block_size=16, num_blocks=10000, append=False, seed=seed, fill=fill)


def sweep_lengths(rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    """Lengths log-uniform in [16, 4096]: floor(exp(U(ln 16, ln 4097))), clipped."""
    x = np.exp(rng.uniform(np.log(16.0), np.log(4097.0), size=num_seqs))
    return np.clip(np.floor(x).astype(np.int64), 16, 4096)


def sweep(block_size: int, head_dim: int, seed: int = 0, num_seqs: int = 512,
          fill: bool = True) -> DecodeWorkload:
    """512 sequences, log-uniform lengths, 32/8 heads, bf16; append then decode.
    Pool = ceil(1.25 * blocks needed after the append) + 1 padding block."""
    rng = np.random.default_rng(seed)
    lens = sweep_lengths(rng, num_seqs)
    need = int(sum(_ceil_div(int(n) + 1, block_size) for n in lens))
    num_blocks = _ceil_div(5 * need, 4) + 1
    return build_private(
        f"sweep_b{block_size}_d{head_dim}", lens, dtype="bf16", num_heads=32, kv_heads=8,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks, append=True, rng=rng,
        seed=seed, fill=fill, meta={"lengths": "log-uniform [16, 4096]"})


SWEEP_CELLS = [(b, d) for b in (16, 32, 64) for d in (64, 128)]


def shared_prefix(seed: int = 0, num_seqs: int = 200, num_beams: int = 16,
                  prefix_tokens: int = 2000, num_blocks: int = 20000,
                  fill: bool = True) -> DecodeWorkload:
    """200 sequences on one shared 2,000-token prefix + private tails; a 16-beam
    fork with copy-on-write of the parent's partly filled last block.

    The decode covers the 200 originals (their cached lengths) and the 16 beams
    (parent length + the one token each beam writes into its private copy).
    """
    rng = np.random.default_rng(seed)
    bs, kv_heads, head_dim, num_heads, dtype = 16, 8, 128, 64, "bf16"
    tails = rng.integers(1, 400, size=num_seqs, endpoint=True)
    pre_lens = prefix_tokens + tails
    pool = BlockPool(num_blocks, rng.permutation(num_blocks))
    padding = pool.take(1)[0]
    prefix_blocks = _ceil_div(prefix_tokens, bs)
    assert prefix_blocks * bs == prefix_tokens, "shared prefix must fill whole blocks"
    shared = pool.take(prefix_blocks)
    tables = []
    for s in range(num_seqs):
        if s > 0:
            pool.share(shared)              # one more table points at the prefix
        tables.append(list(shared) + pool.take(_ceil_div(int(tails[s]), bs)))
    q = _draw(rng, (num_seqs + num_beams, num_heads, head_dim), dtype)
    k_cache = _nan_pool((num_blocks, kv_heads, bs, head_dim), dtype, fill)
    v_cache = _nan_pool((num_blocks, kv_heads, bs, head_dim), dtype, fill)
    if fill:
        _fill_sequence(_stream(seed, 8, 0), k_cache, v_cache, shared, prefix_tokens, dtype)
        _fill_all(seed, 7, k_cache, v_cache, [t[prefix_blocks:] for t in tables], tails, dtype)
    # fork: the first sequence whose last block is only partly filled
    parent = int(np.flatnonzero(pre_lens % bs != 0)[0])
    parent_len = int(pre_lens[parent])
    parent_last = tables[parent][-1]
    fill = parent_len - (len(tables[parent]) - 1) * bs
    fresh = pool.take(num_beams)
    pairs, slots = [], []
    for i in range(num_beams):
        pool.share(tables[parent][:-1])     # beam shares everything but the last block
        tables.append(tables[parent][:-1] + [fresh[i]])
        pairs.append((parent_last, fresh[i]))
        slots.append(fresh[i] * bs + fill)
    k_new = _draw(rng, (num_beams, kv_heads, head_dim), dtype)
    v_new = _draw(rng, (num_beams, kv_heads, head_dim), dtype)
    seq_lens = np.concatenate([pre_lens, np.full(num_beams, parent_len + 1)])
    pre_all = np.concatenate([pre_lens, np.full(num_beams, parent_len)])
    return DecodeWorkload(
        name="shared_prefix", dtype=dtype, num_heads=num_heads, kv_heads=kv_heads,
        head_dim=head_dim, block_size=bs, num_blocks=num_blocks,
        scale=float(1.0 / np.sqrt(head_dim)), q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=_pack_tables(tables, padding),
        seq_lens=seq_lens.astype(np.int32), pre_lens=pre_all.astype(np.int32),
        k_new=k_new, v_new=v_new, slot_mapping=np.asarray(slots, dtype=np.int64),
        append_seq=np.arange(num_seqs, num_seqs + num_beams, dtype=np.int64),
        cow_pairs=np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
        padding_block=int(padding), refcount=pool.refcount.copy(),
        meta={"parent": parent, "shared_blocks": shared, "prefix_blocks": prefix_blocks,
              "num_originals": num_seqs, "num_beams": num_beams, "fresh": fresh,
              "tails": "U{1..400}"})


# --------------------------------------------------------------------------
# prefill workloads: a chunk of queries per sequence, its K/V already cached
# --------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    name: str
    dtype: str
    num_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: np.ndarray                   # [T, Hq, D]: sequence s's chunk is rows query_start[s]..
    k_cache: np.ndarray             # [NB, Hkv, b, D] holding every position, chunk included
    v_cache: np.ndarray
    block_tables: np.ndarray        # int32 [B, max_blocks_per_seq]
    seq_lens: np.ndarray            # int32 [B] cached positions after the chunk's append
    query_lens: np.ndarray          # int32 [B] chunk length (the last query_lens[s] positions)
    padding_block: int
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_queries(self) -> int:
        return int(self.q.shape[0])

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.query_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draw_rows(seed: int, kind: int, shape, dtype: str, rows_per_stream: int = 256) -> np.ndarray:
    """_draw over the leading axis in chunks of rows, chunk i from its own stream
    default_rng([seed, kind, i]), filled in parallel (same result for any
    thread count)."""
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    chunks = range(_ceil_div(shape[0], rows_per_stream))

    def fill(i):
        lo = i * rows_per_stream
        hi = min(shape[0], lo + rows_per_stream)
        out[lo:hi] = _draw(_stream(seed, kind, i), (hi - lo,) + tuple(shape[1:]), dtype)

    with ThreadPoolExecutor(_FILL_THREADS) as ex:
        list(ex.map(fill, chunks))
    return out


def prefill_flops(seq_lens, query_lens, num_heads: int, head_dim: int) -> int:
    """Multiply-adds x 2 of causal prefill: a query at position p scores p + 1
    keys (2*D flops each) and sums as many V rows (2*D), for every query head."""
    total = 0
    for n_ctx, n_q in zip(np.asarray(seq_lens, dtype=np.int64), np.asarray(query_lens, dtype=np.int64)):
        first = int(n_ctx - n_q) + 1                 # keys seen by the chunk's first query
        last = int(n_ctx)
        total += (first + last) * int(n_q) // 2      # sum of an arithmetic run
    return 4 * head_dim * num_heads * total


def build_prefill(name: str, seq_lens, query_lens, *, dtype: str, num_heads: int, kv_heads: int,
                  head_dim: int, block_size: int, num_blocks: int, seed: int = 0,
                  meta: dict | None = None, fixed_tables: dict | None = None) -> PrefillWorkload:
    """Private blocks holding every position (build_private with no append), and
    the chunks' queries, 256 rows per stream default_rng([seed, 13, i])."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    query_lens = np.asarray(query_lens, dtype=np.int64)
    if np.any(query_lens > seq_lens) or np.any(query_lens < 0):
        raise ValueError("a chunk cannot be longer than its sequence")
    base = build_private(name, seq_lens, dtype=dtype, num_heads=num_heads, kv_heads=kv_heads,
                         head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
                         append=False, seed=seed, fixed_tables=fixed_tables)
    q = _draw_rows(seed, 13, (int(query_lens.sum()), num_heads, head_dim), dtype)
    return PrefillWorkload(
        name=name, dtype=dtype, num_heads=num_heads, kv_heads=kv_heads, head_dim=head_dim,
        block_size=block_size, num_blocks=num_blocks, scale=base.scale, q=q,
        k_cache=base.k_cache, v_cache=base.v_cache, block_tables=base.block_tables,
        seq_lens=seq_lens.astype(np.int32), query_lens=query_lens.astype(np.int32),
        padding_block=base.padding_block, meta=dict(meta or {}))


def prefill_tiny(seed: int = 0, head_dim: int = 64, block_size: int = 16,
                 group: int = 4, dtype: str = "bf16") -> PrefillWorkload:
    """Ragged chunks: whole prompts, chunks after a cached prefix, single
    queries, a sequence with no chunk.  2 KV heads."""
    seq_lens = [37, 16, 5, 300, 64, 1, 40, 129]
    query_lens = [37, 9, 5, 70, 1, 1, 0, 129]
    need = sum(_ceil_div(n, block_size) for n in seq_lens)
    return build_prefill("prefill_tiny", seq_lens, query_lens, dtype=dtype,
                         num_heads=2 * group, kv_heads=2, head_dim=head_dim,
                         block_size=block_size, num_blocks=need + 8, seed=seed)


def prefill_tiny_fp32(seed: int = 0) -> PrefillWorkload:
    """The tiny decode shape prefilled: float32, blocks of 4, 8 query / 2 KV
    heads, head_dim 64, pool of 32 blocks, sequences of 10, 1, 16 and 37
    positions with sequence 0 on table [5, 1, 7] (the lihaoran.work example);
    chunks: the whole 10-token prompt, the single token, the last 7 of 16 and
    the last 20 of 37."""
    return build_prefill("prefill_tiny_fp32", [10, 1, 16, 37], [10, 1, 7, 20], dtype="f32",
                         num_heads=8, kv_heads=2, head_dim=64, block_size=4, num_blocks=32,
                         seed=seed, fixed_tables={0: [5, 1, 7]})


def prefill_llama70b(seed: int = 0, num_seqs: int = 32) -> PrefillWorkload:
    """Whole-prompt prefill of 32 chat prompts of U{500..700} tokens (the
    pages' 600-token prompt) on the Llama-3.1-70B layer shape."""
    rng = np.random.default_rng([seed, 17])
    prompt = rng.integers(500, 700, size=num_seqs, endpoint=True)
    need = int(sum(_ceil_div(int(n), 16) for n in prompt))
    return build_prefill("prefill_llama70b", prompt, prompt, dtype="bf16", num_heads=64,
                         kv_heads=8, head_dim=128, block_size=16, num_blocks=need + 64,
                         seed=seed, meta={"prompt": "U{500..700}", "chunk": "whole prompt"})


def prefill_chunked(seed: int = 0, num_seqs: int = 32, chunk: int = 256) -> PrefillWorkload:
    """A 256-token chunk after a cached prefix of U{500..1500} tokens per
    sequence (a prompt continued over reused prefix blocks), 70B layer shape."""
    rng = np.random.default_rng([seed, 19])
    prefix = rng.integers(500, 1500, size=num_seqs, endpoint=True)
    seq_lens = prefix + chunk
    need = int(sum(_ceil_div(int(n), 16) for n in seq_lens))
    return build_prefill("prefill_chunked", seq_lens, [chunk] * num_seqs, dtype="bf16",
                         num_heads=64, kv_heads=8, head_dim=128, block_size=16,
                         num_blocks=need + 64, seed=seed,
                         meta={"prefix": "U{500..1500}", "chunk": chunk})


PREFILL_WORKLOADS = {
    "prefill_tiny": prefill_tiny,
    "prefill_llama70b": prefill_llama70b,
    "prefill_chunked": prefill_chunked,
}


WORKLOADS = {
    "tiny": tiny,
    "llama70b": llama70b,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
    "llama70b_contiguous": llama70b_contiguous,
    "llama70b_tp8": llama70b_tp8,
}


def sweep_name(block_size: int, head_dim: int) -> str:
    return f"sweep_b{block_size}_d{head_dim}"


def make(name: str, seed: int = 0, fill: bool = True) -> DecodeWorkload:
    """Build a workload by name (``sweep_b{16,32,64}_d{64,128}`` for the sweep);
    ``fill=False`` leaves the caches unwritten."""
    if name in WORKLOADS:
        return WORKLOADS[name](seed=seed, fill=fill)
    if name.startswith("sweep_b"):
        b, d = name[len("sweep_b"):].split("_d")
        return sweep(int(b), int(d), seed=seed, fill=fill)
    raise KeyError(f"unknown workload {name!r}")
