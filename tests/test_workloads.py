"""Host-side checks of the seeded workload generators (CPU only)."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_163_amd import workloads as W


def test_bf16_rounding_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5,
                  np.inf, np.nan], dtype=np.float32)
    bits = W.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6);
    # just above a tie rounds up
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F80, 0x7FC0]
    assert list(bits[:7]) == want
    back = oracle.bf16_bits_to_f64(bits[:6])
    assert np.array_equal(back[:5], [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5])


def test_tiny_matches_its_description():
    w = W.tiny()
    assert w.dtype == "f32" and w.q.dtype == np.float32
    assert list(w.pre_lens) == [10, 1, 16, 37] and list(w.seq_lens) == [11, 2, 17, 38]
    assert list(w.block_tables[0, :3]) == [5, 1, 7]
    assert (w.num_heads, w.kv_heads, w.head_dim, w.block_size, w.num_blocks) == (8, 2, 64, 4, 32)
    assert w.k_cache.shape == (32, 2, 4, 64)
    # each sequence's blocks are distinct, no block shared between sequences
    used = []
    for s in range(4):
        nb = oracle.block_layout(int(w.seq_lens[s]), 4)[0]
        used += list(w.block_tables[s, :nb])
    assert len(used) == len(set(used)) and w.padding_block not in used
    # sequence 2 (16 cached) takes a fresh block for its 17th token
    assert oracle.block_layout(16, 4)[0] == 4 and oracle.block_layout(17, 4)[0] == 5
    # slot of seq 0's new token: position 10 -> block 7, slot 2
    assert w.slot_mapping[0] == 7 * 4 + 2
    # poison: everything not live is NaN
    live = np.zeros((32, 4), dtype=bool)
    for s in range(4):
        for t in range(int(w.pre_lens[s])):
            p, o = oracle.translate(w.block_tables[s], t, 4)
            live[p, o] = True
    kt = w.k_cache.transpose(0, 2, 1, 3)
    assert np.all(np.isfinite(kt[live])) and np.all(np.isnan(kt[~live]))


def test_generation_is_deterministic_and_thread_independent(monkeypatch):
    a = W.sweep(16, 64, num_seqs=24)
    monkeypatch.setattr(W, "_FILL_THREADS", 1)
    b = W.sweep(16, 64, num_seqs=24)
    for f in ("q", "k_cache", "v_cache", "block_tables", "seq_lens", "slot_mapping", "k_new"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_llama70b_shape_and_lengths():
    w = W.llama70b()
    assert (w.num_heads, w.kv_heads, w.head_dim, w.block_size, w.num_blocks) == (64, 8, 128, 16, 20000)
    assert w.num_seqs == 256 and w.dtype == "bf16" and w.k_cache.dtype == np.uint16
    assert w.pre_lens.min() >= 500 and w.pre_lens.max() <= 950
    assert np.array_equal(w.seq_lens, w.pre_lens + 1)
    assert w.max_blocks_per_seq <= 60
    nb = [oracle.block_layout(int(n), 16)[0] for n in w.seq_lens]
    ids = np.concatenate([w.block_tables[s, :nb[s]] for s in range(256)])
    assert len(np.unique(ids)) == len(ids)
    assert np.all((ids >= 0) & (ids < 20000))
    # the benchmark's byte numerator: live tokens only
    assert W.decode_kv_bytes(w.seq_lens, 8, 128, 2) == int(w.seq_lens.sum()) * 4096


def test_shared_prefix_refcounts_and_fork():
    w = W.shared_prefix()
    m = w.meta
    shared = m["shared_blocks"]
    assert len(shared) == 125 and m["num_originals"] == 200 and m["num_beams"] == 16
    # every original and every beam points at the same 125 prefix blocks
    assert np.all(w.block_tables[:, :125] == np.asarray(shared)[None, :])
    assert np.all(w.refcount[shared] == 216)
    parent = m["parent"]
    plen = int(w.pre_lens[parent])
    assert plen % 16 != 0
    last = oracle.block_layout(plen, 16)[0] - 1
    parent_last = int(w.block_tables[parent, last])
    assert np.all(w.cow_pairs[:, 0] == parent_last)
    assert np.array_equal(w.cow_pairs[:, 1], w.block_tables[200:, last])
    assert len(set(w.cow_pairs[:, 1])) == 16
    # footprint: prefix + private tails + one copied block per beam
    private = sum(oracle.block_layout(int(n) - 2000, 16)[0] for n in w.pre_lens[:200])
    assert w.refcount[w.padding_block] == 1          # held by the allocator, never read
    assert int((w.refcount > 0).sum()) == 125 + private + 16 + 1
    assert list(w.seq_lens[200:]) == [plen + 1] * 16
    # the beams' new tokens go to the slot after the parent's last token, in the copies
    for i in range(16):
        blk, off = divmod(int(w.slot_mapping[i]), 16)
        assert blk == w.cow_pairs[i, 1] and off == plen - last * 16


def test_long_context_and_sweep_shapes():
    w = W.long_context()
    assert w.num_seqs == 16 and np.all(w.seq_lens == 8192) and w.max_blocks_per_seq == 512
    assert w.slot_mapping.size == 0
    lens = W.sweep_lengths(np.random.default_rng(0), 4096)
    assert lens.min() >= 16 and lens.max() <= 4096
    # log-uniform: the median sits near the geometric mean of the ends (256)
    assert 200 < np.median(lens) < 330


@pytest.mark.parametrize("b,d", W.SWEEP_CELLS)
def test_sweep_cells_small(b, d):
    w = W.sweep(b, d, num_seqs=16)
    assert (w.block_size, w.head_dim, w.num_heads, w.kv_heads) == (b, d, 32, 8)
    need = sum(oracle.block_layout(int(n), b)[0] for n in w.seq_lens)
    assert w.num_blocks == -(-5 * need // 4) + 1


def test_prefill_workloads_shapes_and_determinism():
    w = W.prefill_tiny()
    assert w.num_queries == int(w.query_lens.sum())
    assert list(w.query_start) == [0] + list(np.cumsum(w.query_lens))
    assert np.all(w.query_lens <= w.seq_lens)
    assert w.q.shape == (w.num_queries, w.num_heads, w.head_dim) and w.q.dtype == np.uint16
    # every position of every sequence is cached; slots past the end hold NaN
    for s, n in enumerate(w.seq_lens):
        blocks, unused = oracle.block_layout(int(n), w.block_size)
        if unused:
            last = w.block_tables[s, blocks - 1]
            assert np.all(w.k_cache[last, :, w.block_size - unused:, :] == W.BF16_NAN)
    again = W.prefill_tiny()
    assert np.array_equal(again.q, w.q) and np.array_equal(again.k_cache, w.k_cache)
    big = W.prefill_llama70b(num_seqs=4)
    assert np.array_equal(big.query_lens, big.seq_lens)
    assert big.seq_lens.min() >= 500 and big.seq_lens.max() <= 700
    ch = W.prefill_chunked(num_seqs=4)
    assert np.all(ch.query_lens == 256) and np.all(ch.seq_lens >= 756)


def test_prefill_flops_counts_causal_pairs():
    lens, nq = [5, 9, 1], [5, 3, 1]
    pairs = sum(p + 1 for n, c in zip(lens, nq) for p in range(n - c, n))
    assert W.prefill_flops(lens, nq, num_heads=4, head_dim=8) == 4 * 8 * 4 * pairs


def test_unique_kv_bytes_counts_shared_blocks_once():
    bt = np.array([[3, 4, 0], [3, 5, 0], [6, 0, 0]], dtype=np.int32)
    # b = 4; seqs share block 3 (full); block 4 holds 2 live slots, 5 holds 3, 6 holds 1
    lens = np.array([6, 7, 1], dtype=np.int32)
    per_token = 2 * 2 * 8 * 2                    # K+V, 2 KV heads, D = 8, bf16
    assert W.unique_kv_bytes(bt, lens, 4, 2, 8, 2) == (4 + 2 + 3 + 1) * per_token
    assert W.decode_kv_bytes(lens, 2, 8, 2) == 14 * per_token
    w = W.tiny()
    assert W.unique_kv_bytes(w.block_tables, w.seq_lens, w.block_size, w.kv_heads, w.head_dim,
                             w.elem_bytes) == W.decode_kv_bytes(w.seq_lens, w.kv_heads,
                                                                w.head_dim, w.elem_bytes)
