"""The decode step captured in a HIP graph (through torch's graph API) and
replayed: the KV append, the decode through pa_decode_noalloc (partials in
the library's static scratch: the entry point for callers that cannot
allocate, graph capture among them) and the ordered decode with a workspace
allocated before the capture.  No call of the step records a memset or an
allocation, so every replay must reproduce the eager step byte for byte,
also with eager calls between the replays that reuse the same scratch.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from paged_kv_cache_163_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_ATOL, BF16_RTOL = 1e-2, 2e-2


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
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_decode_step_replays_from_a_graph(pa):
    # split sequences (256-token partitions: the reduce kernel and the scratch
    # are in play), a one-token sequence and a full last block
    lens = [300, 1000, 2047, 17, 1, 512]
    w = W.build_private("graph", lens, dtype="bf16", num_heads=32, kv_heads=4, head_dim=128,
                        block_size=16, num_blocks=sum(-(-n // 16) + 1 for n in lens) + 4,
                        append=True, seed=21)
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    q, bt, ln = dev(w.q), dev(w.block_tables), dev(w.seq_lens)
    k_new, v_new, slots = dev(w.k_new), dev(w.v_new), dev(w.slot_mapping)
    order = pa.longest_first(ln)
    P, mx = 256, int(w.max_seq_len)
    out_na, out_ord = torch.empty_like(q), torch.empty_like(q)
    plan = pa.decode_plan(w.num_seqs, w.num_heads, w.kv_heads, w.head_dim, w.block_size, mx, P,
                          q.dtype, "auto")
    assert plan.num_partitions > 1
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=DEV)

    def step():
        pa.kv_append(k_new, v_new, kc, vc, slots)
        pa.decode_noalloc(q, kc, vc, bt, ln, w.scale, max_seq_len=mx, partition_size=P,
                          out=out_na)
        pa.decode_ordered(q, kc, vc, bt, ln, order, w.scale, max_seq_len=mx, partition_size=P,
                          out=out_ord, workspace=ws)

    # eager step, checked against the oracle
    step()
    torch.cuda.synchronize()
    want_na, want_ord = out_na.clone(), out_ord.clone()
    kref, vref = w.k_cache.copy(), w.v_cache.copy()
    oracle.kv_append(kref, vref, w.k_new, w.v_new, w.slot_mapping, w.block_size)
    ref = oracle.paged_decode(w.q, kref, vref, w.block_tables, w.seq_lens, w.scale, w.block_size)
    got = oracle.to_f64(want_na.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(np.abs(got - ref) <= BF16_ATOL + BF16_RTOL * np.abs(ref))
    assert torch.equal(bits(want_na), bits(want_ord))

    # capture (warm-up on the capture stream first, as torch asks)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    # replays, with eager work between them: an eager no-alloc decode of
    # other inputs (the same scratch) and garbage written into the outputs
    other_q = torch.randn_like(q.float()).to(q.dtype)
    other_out = torch.empty_like(q)
    for r in range(5):
        out_na.fill_(float("nan"))
        out_ord.fill_(float("nan"))
        pa.decode_noalloc(other_q, kc, vc, bt, ln, w.scale, max_seq_len=mx, partition_size=P,
                          out=other_out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out_na), bits(want_na)), f"replay {r}: pa_decode_noalloc"
        assert torch.equal(bits(out_ord), bits(want_ord)), f"replay {r}: pa_decode_ordered"
