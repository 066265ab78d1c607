"""Seeded random configurations against the oracle, every output element.

Each case draws its own shape from numpy.random.default_rng([20261202, kind,
case]): batch size, ragged lengths (some empty), block size, KV heads, group
size, head dim, dtype and partition size.  It then runs every kernel that
supports the shape through the C ABI, and the pinned float64 oracle computes
the reference from the same bytes.

PA_RANDOM_SCALE=k (environment) runs k times as many cases of each kind
(new seeds after the default ones), for a wider sweep.

Bars as in test_gpu_parity.py:
* copy-on-write copies and appends are bit-exact;
* fp32 outputs within 1e-5 absolute;
* bf16 outputs within 1e-2 + 2e-2 |ref|.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from paged_kv_cache_163_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = max(1, int(os.environ.get("PA_RANDOM_SCALE", "1")))


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


def host(t):
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def raw(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_close(got, ref, dtype, what):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-5, f"{what}: max abs err {err.max():.3g}"
    else:
        bad = err > 1e-2 + 2e-2 * np.abs(ref)
        assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, max {err.max():.3g}"


def draw_lengths(rng, n, longest):
    """Ragged lengths: about one in ten empty, the rest log-uniform in [1, longest]."""
    lens = np.floor(np.exp(rng.uniform(0.0, np.log(longest + 1), size=n))).astype(np.int64)
    lens = np.clip(lens, 1, longest)
    lens[rng.random(n) < 0.1] = 0
    return lens


@pytest.mark.parametrize("case", range(40 * SCALE))
def test_random_decode_step(pa, case):
    rng = np.random.default_rng([20261202, 1, case])
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    head_dim = int(rng.choice([64, 128]))
    kv_heads = int(rng.integers(1, 5))
    group = int(rng.choice([1, 2, 4, 8] if dtype == "f32" else [1, 2, 4, 8, 16]))
    block_size = int(rng.choice([1, 4, 8, 16, 32, 64] if dtype == "f32" else [16, 32, 64]))
    pre = draw_lengths(rng, int(rng.integers(1, 25)), 1500)
    nb = int(sum(-(-(int(n) + 1) // block_size) for n in pre)) + 8
    w = W.build_private("random", pre, dtype=dtype, num_heads=kv_heads * group,
                        kv_heads=kv_heads, head_dim=head_dim, block_size=block_size,
                        num_blocks=nb, append=True, seed=1000 + case)
    # copy-on-write of up to two sequences' last blocks into free blocks
    free = sorted(set(range(nb)) - set(w.block_tables.ravel().tolist()))
    srcs = [int(w.block_tables[s, -(-int(pre[s]) // block_size) - 1])
            for s in range(len(pre)) if pre[s] > 0][:2]
    pairs = np.array([[b, free[i]] for i, b in enumerate(srcs)], dtype=np.int64).reshape(-1, 2)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.copy_blocks(kc, vc, pairs)
    oracle.kv_append(kc, vc, w.k_new, w.v_new, w.slot_mapping, block_size)
    k, v = dev(w.k_cache), dev(w.v_cache)
    if pairs.shape[0]:
        pa.copy_blocks(k, v, dev(pairs))
    pa.kv_append(dev(w.k_new), dev(w.v_new), k, v, dev(w.slot_mapping))
    torch.cuda.synchronize()
    assert np.array_equal(raw(host(k)), raw(kc)) and np.array_equal(raw(host(v)), raw(vc))
    ref = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale, block_size)
    part = int(rng.choice([0, 0, 16, 32, 96, 512, 4096]))
    kernels = ["valu"] if dtype == "f32" else ["mfma"]
    if dtype == "bf16" and group <= 8:
        kernels.append("valu")
    q, bt, lens = dev(w.q), dev(w.block_tables), dev(w.seq_lens)
    what = (f"case {case}: {dtype} D={head_dim} Hkv={kv_heads} G={group} b={block_size} "
            f"B={len(pre)} P={part}")
    for kernel in kernels:
        out = pa.decode(q, k, v, bt, lens, w.scale, max_seq_len=w.max_seq_len, kernel=kernel,
                        partition_size=part)
        torch.cuda.synchronize()
        assert_close(oracle.to_f64(host(out)), ref, dtype, f"{what} {kernel}")


@pytest.mark.parametrize("case", range(15 * SCALE))
def test_random_prefill(pa, case):
    rng = np.random.default_rng([20261202, 2, case])
    head_dim = int(rng.choice([64, 128]))
    kv_heads = int(rng.integers(1, 4))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    block_size = int(rng.choice([16, 32, 64]))
    lens = np.maximum(draw_lengths(rng, int(rng.integers(1, 13)), 700), 1)
    chunks = np.minimum(lens, draw_lengths(rng, len(lens), 300))
    nb = int(sum(-(-int(n) // block_size) for n in lens)) + 8
    w = W.build_prefill("random", lens, chunks, dtype="bf16", num_heads=kv_heads * group,
                        kv_heads=kv_heads, head_dim=head_dim, block_size=block_size,
                        num_blocks=nb, seed=2000 + case)
    ref = oracle.paged_prefill(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                               w.query_lens, w.scale, block_size)
    if w.num_queries == 0:
        return
    out = pa.prefill(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables),
                     dev(w.seq_lens), dev(w.query_start), w.scale,
                     max_query_len=int(w.query_lens.max()))
    torch.cuda.synchronize()
    assert_close(oracle.to_f64(host(out)), ref, "bf16",
                 f"case {case}: D={head_dim} Hkv={kv_heads} G={group} b={block_size} "
                 f"chunks={chunks.tolist()} lens={lens.tolist()}")


@pytest.mark.parametrize("case", range(10 * SCALE))
def test_random_prefill_vector_alu(pa, case):
    """Prefill shapes the matrix-core kernel does not take: float32 at any
    power-of-two block size, bf16 at blocks below 16."""
    rng = np.random.default_rng([20261202, 5, case])
    dtype = str(rng.choice(["f32", "bf16"]))
    head_dim = int(rng.choice([64, 128]))
    kv_heads = int(rng.integers(1, 4))
    group = int(rng.choice([1, 2, 4, 8]))
    block_size = int(rng.choice([1, 2, 4, 8, 16, 32] if dtype == "f32" else [1, 2, 4, 8]))
    lens = np.maximum(draw_lengths(rng, int(rng.integers(1, 9)), 300), 1)
    chunks = np.minimum(lens, draw_lengths(rng, len(lens), 120))
    nb = int(sum(-(-int(n) // block_size) for n in lens)) + 8
    w = W.build_prefill("random_valu", lens, chunks, dtype=dtype, num_heads=kv_heads * group,
                        kv_heads=kv_heads, head_dim=head_dim, block_size=block_size,
                        num_blocks=nb, seed=5000 + case)
    if w.num_queries == 0:
        return
    ref = oracle.paged_prefill(w.q, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                               w.query_lens, w.scale, block_size)
    out = pa.prefill(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_tables),
                     dev(w.seq_lens), dev(w.query_start), w.scale,
                     max_query_len=int(w.query_lens.max()))
    torch.cuda.synchronize()
    assert_close(oracle.to_f64(host(out)), ref, dtype,
                 f"case {case}: {dtype} D={head_dim} Hkv={kv_heads} G={group} b={block_size} "
                 f"chunks={chunks.tolist()} lens={lens.tolist()}")


@pytest.mark.parametrize("case", range(15 * SCALE))
def test_random_shared_prefix(pa, case):
    rng = np.random.default_rng([20261202, 3, case])
    head_dim = int(rng.choice([64, 128]))
    kv_heads = int(rng.integers(1, 4))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    block_size = int(rng.choice([16, 32, 64]))
    B = int(rng.integers(1, 21))
    # adjacent groups of random sizes with random prefix lengths (whole blocks);
    # members reach past their prefix
    cuts = np.sort(rng.choice(np.arange(1, B), size=min(B - 1, int(rng.integers(0, 4))),
                              replace=False)) if B > 1 else np.array([], dtype=np.int64)
    bounds = [0] + cuts.tolist() + [B]
    prefix = [int(rng.integers(0, 6)) for _ in range(len(bounds) - 1)]
    lens = np.zeros(B, dtype=np.int64)
    for g in range(len(prefix)):
        for s in range(bounds[g], bounds[g + 1]):
            lens[s] = prefix[g] * block_size + int(draw_lengths(rng, 1, 400)[0])
    nb = int(sum(-(-int(n) // block_size) for n in lens)) + 8
    w = W.build_private("random_shared", lens, dtype="bf16", num_heads=kv_heads * group,
                        kv_heads=kv_heads, head_dim=head_dim, block_size=block_size,
                        num_blocks=nb, append=False, seed=3000 + case)
    bt = w.block_tables.copy()
    for g in range(len(prefix)):
        s0 = bounds[g]
        for s in range(s0 + 1, bounds[g + 1]):
            bt[s, :prefix[g]] = bt[s0, :prefix[g]]
    ref = oracle.paged_decode(w.q, w.k_cache, w.v_cache, bt, w.seq_lens, w.scale, block_size)
    ppart = int(rng.choice([0, 32, 64, 96]))
    out = pa.decode_shared_prefix(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(bt),
                                  dev(w.seq_lens), w.scale, bounds, prefix,
                                  max_seq_len=w.max_seq_len, prefix_partition_size=ppart)
    torch.cuda.synchronize()
    assert_close(oracle.to_f64(host(out)), ref, "bf16",
                 f"case {case}: D={head_dim} Hkv={kv_heads} G={group} b={block_size} "
                 f"groups={bounds} prefix={prefix} P={ppart}")
    # the tails in a random order: the same bytes
    order = torch.from_numpy(rng.permutation(B).astype(np.int32)).to(DEV)
    again = pa.decode_shared_prefix(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(bt),
                                    dev(w.seq_lens), w.scale, bounds, prefix,
                                    max_seq_len=w.max_seq_len, prefix_partition_size=ppart,
                                    order=order)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out.view(torch.int16)), f"case {case}: order"


@pytest.mark.parametrize("case", range(20 * SCALE))
def test_random_fused_append(pa, case):
    """pa_decode_append: one new token per sequence (slot -1 for about one
    sequence in five, whose length then stays put), appended and decoded in
    one launch.  The cache must match the oracle's append bit for bit."""
    rng = np.random.default_rng([20261202, 4, case])
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    head_dim = int(rng.choice([64, 128]))
    kv_heads = int(rng.integers(1, 5))
    group = int(rng.choice([1, 2, 4, 8] if dtype == "f32" else [1, 2, 4, 8, 16]))
    block_size = int(rng.choice([1, 4, 16, 32] if dtype == "f32" else [16, 32, 64]))
    pre = draw_lengths(rng, int(rng.integers(1, 25)), 1500)
    nb = int(sum(-(-(int(n) + 1) // block_size) for n in pre)) + 8
    w = W.build_private("random_fused", pre, dtype=dtype, num_heads=kv_heads * group,
                        kv_heads=kv_heads, head_dim=head_dim, block_size=block_size,
                        num_blocks=nb, append=True, seed=4000 + case)
    k_new, v_new, slots = W.per_sequence_append(w)
    skip = rng.random(len(pre)) < 0.2
    slots[skip] = -1
    lens = np.where(skip, w.pre_lens, w.seq_lens).astype(np.int32)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(kc, vc, k_new[~skip], v_new[~skip], slots[~skip], block_size)
    ref = oracle.paged_decode(w.q, kc, vc, w.block_tables, lens, w.scale, block_size)
    part = int(rng.choice([0, 0, 16, 32, 96, 512]))
    kernels = ["valu"] if dtype == "f32" else ["mfma"] + (["valu"] if group <= 8 else [])
    what = (f"case {case}: {dtype} D={head_dim} Hkv={kv_heads} G={group} b={block_size} "
            f"B={len(pre)} P={part}")
    for kernel in kernels:
        k, v = dev(w.k_cache), dev(w.v_cache)
        out = pa.decode_append(dev(w.q), k, v, dev(k_new), dev(v_new), dev(slots),
                               dev(w.block_tables), dev(lens), w.scale,
                               max_seq_len=int(lens.max()), partition_size=part, kernel=kernel)
        torch.cuda.synchronize()
        assert np.array_equal(raw(host(k)), raw(kc)) and np.array_equal(raw(host(v)), raw(vc)), \
            f"{what} {kernel}: cache"
        assert_close(oracle.to_f64(host(out)), ref, dtype, f"{what} {kernel}")
        # pa_decode_append_ordered in a random order: the same cache and the
        # same outputs bit for bit
        order = torch.from_numpy(rng.permutation(len(pre)).astype(np.int32)).to(DEV)
        k, v = dev(w.k_cache), dev(w.v_cache)
        again = pa.decode_append(dev(w.q), k, v, dev(k_new), dev(v_new), dev(slots),
                                 dev(w.block_tables), dev(lens), w.scale,
                                 max_seq_len=int(lens.max()), partition_size=part, kernel=kernel,
                                 order=order)
        torch.cuda.synchronize()
        assert np.array_equal(raw(host(k)), raw(kc)) and np.array_equal(raw(host(v)), raw(vc)), \
            f"{what} {kernel} ordered: cache"
        assert torch.equal(again.view(torch.int32 if dtype == "f32" else torch.int16),
                           out.view(torch.int32 if dtype == "f32" else torch.int16)), \
            f"{what} {kernel}: ordered"
