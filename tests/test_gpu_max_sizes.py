"""Parity at the size limits of the C ABI.

* A pool larger than 4 GiB per cache: the blocks of a small batch are moved to
  ids at and above 2^17, whose byte offsets (32 KiB blocks at the 70B layer
  shape) lie past 4 GiB, so every kernel's address arithmetic must be 64-bit.
  Decode (all three kernels), append, copy-on-write, prefill and the
  shared-prefix decode are compared with the oracle run on the small pool.
* One 262,144-token sequence: the split kernels at thousands of partitions,
  up to the 16,384-partition limit of the merge, which is refused beyond it.

Bars as in test_gpu_parity.py: bit-exact writes; bf16 outputs within
1e-2 + 2e-2 |ref| of the float64 oracle.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from paged_kv_cache_163_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HIGH = 1 << 17   # first relocated block id: 2^17 blocks x 32 KiB = 4 GiB


@pytest.fixture(scope="module")
def pa(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_163_amd import pa as binding
    return binding


def dev(arr):
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(arr).to(DEV)


def bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(t):
    return oracle.to_f64(bits(t))


def assert_close(got, ref, what=""):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > 1e-2 + 2e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max {err.max():.3g}"


def big_pool(k_small, v_small):
    """Device caches of HIGH + n blocks (NaN below HIGH) holding the small
    pool's blocks at ids HIGH + i."""
    n = k_small.shape[0]
    shape = (HIGH + n,) + k_small.shape[1:]
    k = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    v = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    k[HIGH:] = dev(k_small)
    v[HIGH:] = dev(v_small)
    assert k[HIGH].data_ptr() - k.data_ptr() >= 1 << 32
    return k, v


def test_pool_beyond_4gib_every_call(pa):
    w = W.build_private("far", [1, 100, 700, 33, 257], dtype="bf16", num_heads=64, kv_heads=8,
                        head_dim=128, block_size=16, num_blocks=80, append=True, seed=3)
    k, v = big_pool(w.k_cache, w.v_cache)
    bt = dev(w.block_tables + HIGH)
    # copy-on-write of sequence 2's last block into a free block, then the appends
    free = sorted(set(range(w.num_blocks)) - set(w.block_tables.ravel().tolist()))
    pairs = np.array([[w.block_tables[2, 43], free[0]]], dtype=np.int64)
    pa.copy_blocks(k, v, dev(pairs + HIGH))
    pa.kv_append(dev(w.k_new), dev(w.v_new), k, v, dev(w.slot_mapping + HIGH * w.block_size))
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.copy_blocks(kc, vc, pairs)
    oracle.kv_append(kc, vc, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k[HIGH:]), kc) and np.array_equal(bits(v[HIGH:]), vc)
    assert bool(torch.isnan(k[:HIGH]).all())                    # nothing written below
    ref = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale, w.block_size)
    lens, q = dev(w.seq_lens), dev(w.q)
    for kernel, part in (("mfma", 0), ("mfma", 64), ("valu", 0)):
        out = pa.decode(q, k, v, bt, lens, w.scale, max_seq_len=w.max_seq_len, kernel=kernel,
                        partition_size=part)
        torch.cuda.synchronize()
        assert_close(as_f64(out), ref, f"decode {kernel} P={part}")
    # shared-prefix decode: sequences 1..3 share sequence 1's first two blocks
    bt2 = w.block_tables.copy()
    bt2[2:4, :2] = bt2[1, :2]
    ref2 = oracle.paged_decode(w.q, kc, vc, bt2, w.seq_lens, w.scale, w.block_size)
    out = pa.decode_shared_prefix(q, k, v, dev(bt2 + HIGH), lens, w.scale, [1, 4], [2],
                                  max_seq_len=w.max_seq_len, prefix_partition_size=32)
    torch.cuda.synchronize()
    assert_close(as_f64(out), ref2, "shared-prefix decode")
    # prefill: chunks at the end of each sequence, over the appended pool
    qlens = np.array([1, 37, 300, 33, 0], dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    qp = W._draw(np.random.default_rng(5), (int(qlens.sum()), 64, 128), "bf16")
    pref = oracle.paged_prefill(qp, kc, vc, w.block_tables, w.seq_lens, qlens, w.scale,
                                w.block_size)
    out = pa.prefill(dev(qp), k, v, bt, lens, dev(starts), w.scale, max_query_len=300)
    torch.cuda.synchronize()
    assert_close(as_f64(out), pref, "prefill")


def test_longest_sequence_up_to_the_partition_limit(pa):
    L = 1 << 18
    w = W.build_private("long1", [L, 5], dtype="bf16", num_heads=8, kv_heads=1, head_dim=128,
                        block_size=16, num_blocks=L // 16 + 8, append=False, seed=4)
    ref = oracle.paged_decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens, w.scale, 16)
    d = dict(q=dev(w.q), k=dev(w.k_cache), v=dev(w.v_cache), bt=dev(w.block_tables),
             lens=dev(w.seq_lens))
    cases = (("mfma", 0), ("mfma", 32), ("valu", 16))
    for kernel, part in cases:
        plan = pa.decode_plan(2, 8, 1, 128, 16, L, part, torch.bfloat16, kernel)
        if kernel == "valu":
            assert plan.num_partitions == 16384                 # the merge's limit
        out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["lens"], w.scale, max_seq_len=L,
                        partition_size=part, kernel=kernel)
        torch.cuda.synchronize()
        assert_close(as_f64(out), ref, f"{kernel} P={part} ({plan.num_partitions} partitions)")
    with pytest.raises(NotImplementedError):                     # 32,768 partitions
        pa.decode(d["q"], d["k"], d["v"], d["bt"], d["lens"], w.scale, max_seq_len=L,
                  partition_size=8, kernel="valu")
