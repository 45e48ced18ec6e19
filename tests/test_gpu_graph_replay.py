"""Every attention and producer entry point captured in a HIP graph (torch.cuda.CUDAGraph
on the capture stream) and replayed several times, with eager work of the library between
the replays: each replay must give the eager call's outputs bit for bit. The kernels use
no atomics and no reduction whose order depends on timing, so the same launch gives the
same bits; before each replay the outputs are overwritten with a sentinel and a cache the
call writes is restored to its state before the call, so a launch that a replay skipped
shows up as a mismatch."""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import DecodeSetup, PrefillSetup, bf16_tensor, gpu_cache, need_gpu, say, up

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _cache_tensors(c):
    return (c.k_cache, c.v_cache, c.k_scale, c.v_scale)


def _sentinel(t: torch.Tensor):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(0x5A)


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return bool(torch.equal(a.contiguous().reshape(-1).view(torch.uint8),
                            b.contiguous().reshape(-1).view(torch.uint8)))


def _replay_check(name, run, caches=()):
    """run() launches the entry point and returns its output tensors. caches: PagedCaches
    that run() writes; they are put back to their state before the call ahead of each
    eager run and each replay."""
    torch.cuda.synchronize()
    before = [[t.clone() for t in _cache_tensors(c)] for c in caches]

    def restore():
        for c, snap in zip(caches, before):
            for t, s in zip(_cache_tensors(c), snap):
                t.copy_(s)

    ref = [t.clone() for t in run()]
    ref_cache = [[t.clone() for t in _cache_tensors(c)] for c in caches]
    torch.cuda.synchronize()

    # warm the capture path on a side stream, as torch asks, then capture
    restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    restore()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        restore()
        run()                       # eager work between the replays
        torch.cuda.synchronize()
        for t in outs:
            _sentinel(t)
        restore()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same_bits(a, b), f"{name}: replay {r} output {i} differs from the eager call"
        for c, rc in zip(caches, ref_cache):
            for i, (a, b) in enumerate(zip(_cache_tensors(c), rc)):
                assert _same_bits(a, b), f"{name}: replay {r} cache array {i} differs"
    say(f"  {name}: {REPLAYS} replays bit-identical to the eager call")
    del g


@pytest.mark.parametrize("n_seqs", [3, 20])
def test_graph_decode_verify_int8p(n_seqs):
    # 3 sequences: the (partition, head, sequence) grid; 20: the flattened grid of work items
    need_gpu()
    rng = np.random.default_rng(700 + n_seqs)
    ctx = [int(x) for x in rng.integers(1, 3000, n_seqs)]
    ctx[0] = 2049
    say(f"graph replay, decode family, contexts {ctx}")
    st = DecodeSetup(workloads.make_decode_case(700 + n_seqs, ctx, pages="random", k_outliers=4,
                                                q_rows_per_seq=4))
    mx = int(st.case.max_context_len)
    ws = torch.empty(lib.attn_decode_workspace_bytes(n_seqs, mx, 24), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((n_seqs, 24, 256), dtype=torch.float32, device="cuda")
    _replay_check("attn_decode (workspace given)",
                  lambda: (lib.attn_decode(st.q, st.cache, st.table, st.ctx, mx, out=out,
                                           workspace=ws),))
    _replay_check("attn_decode (workspace allocated in the call)",
                  lambda: (lib.attn_decode(st.q, st.cache, st.table, st.ctx, mx),))
    _replay_check("attn_verify nq=4",
                  lambda: (lib.attn_verify(st.q_all, st.cache, st.table, st.ctx, mx),))
    _replay_check("attn_decode_int8p nq=4",
                  lambda: (lib.attn_decode_int8p(st.q_all, st.cache, st.table, st.ctx, mx),))
    _replay_check("attn_decode_int8p one row, 128-key partitions",
                  lambda: (lib.attn_decode_int8p(st.q, st.cache, st.table, st.ctx, mx,
                                                 partition_rows=128),))
    nq_out = torch.empty((n_seqs, 24, 256), dtype=torch.float32, device="cuda")
    _replay_check("attn_decode_noalloc",
                  lambda: (lib.attn_decode_noalloc(st.q, st.cache, st.table, st.ctx, mx,
                                                   out=nq_out),))
    qc, qs = lib.q_quant(st.q)
    _replay_check("attn_decode_q8",
                  lambda: (lib.attn_decode(qc, st.cache, st.table, st.ctx, mx, q_scales=qs),))


@pytest.mark.parametrize("ctx,n_new", [(1000, 300), (700, 5), (700, 40)])
def test_graph_prefill_chunk(ctx, n_new):
    need_gpu()
    say(f"graph replay, prefill chunk ctx={ctx} n_new={n_new}")
    st = PrefillSetup(workloads.make_prefill_case(710 + n_new, ctx, n_new, pages="random",
                                                  k_outliers=4))
    _replay_check("attn_prefill_chunk causal",
                  lambda: (lib.attn_prefill_chunk(st.q, st.cache, st.table, ctx, True),))
    _replay_check("attn_prefill_chunk full",
                  lambda: (lib.attn_prefill_chunk(st.q, st.cache, st.table, ctx, False),))
    _replay_check("attn_prefill_chunk_split causal",
                  lambda: (lib.attn_prefill_chunk_split(st.q, st.cache, st.table, ctx, True),))


@pytest.mark.parametrize("n", [300, 2048])
def test_graph_chunk_bf16(n):
    need_gpu()
    say(f"graph replay, bf16 first chunk n={n}")
    rng = np.random.default_rng(720 + n)
    q, k, v = (bf16_tensor(workloads.f32_to_bf16_bits(
        rng.standard_normal((n, h, 256), dtype=np.float32))) for h in (24, 4, 4))
    _replay_check("attn_chunk_bf16 split",
                  lambda: (lib.attn_chunk_bf16(q, k, v, causal=True),))
    _replay_check("attn_chunk_bf16 one pass",
                  lambda: (lib.attn_chunk_bf16(q, k, v, causal=True, split=False),))


def test_graph_writers():
    need_gpu()
    say("graph replay, kv_quant_write / q_quant / kv_produce")
    case = workloads.make_producer_case(730, 300, start=5, rotary_dim=256)
    q, k, v = case.data()
    table = up(case.table())
    pos, slots = up(case.positions), up(case.slots)
    cache = gpu_cache(case.num_pages, 4)
    tk, tv = up(k), up(v)
    qb, kb, vb = (bf16_tensor(workloads.f32_to_bf16_bits(a)) for a in (q, k, v))
    _replay_check("kv_quant_write fp32",
                  lambda: (lib.kv_quant_write(tk, tv, slots, cache) or ()), caches=(cache,))
    _replay_check("q_quant", lambda: lib.q_quant(qb))
    _replay_check("kv_produce bf16 -> q codes",
                  lambda: lib.kv_produce(qb, kb, vb, pos, table, slots, cache), caches=(cache,))
    _replay_check("kv_produce bf16 -> rotated rows",
                  lambda: lib.kv_produce(qb, kb, vb, pos, table, slots, cache,
                                         rotated_bf16=True), caches=(cache,))


def test_graph_prefill_step():
    # a first chunk (bf16 route), then a chunk with history (int8 route): the graph of the
    # second call re-runs the producer into the restored cache and the attention over it
    need_gpu()
    say("graph replay, prefill_step first chunk and a chunk with history")
    full = workloads.make_producer_case(740, 400, start=0, rotary_dim=256)
    q, k, v = full.data()
    qb, kb, vb = (bf16_tensor(workloads.f32_to_bf16_bits(a)) for a in (q, k, v))
    table = up(full.table())
    cache = gpu_cache(full.num_pages, 4)
    row = up((full.slots[::16] // 16).astype(np.int32))
    pos, slots = up(full.positions), up(full.slots)
    a = slice(0, 250)
    b = slice(250, 400)
    _replay_check("prefill_step first chunk",
                  lambda: (lib.prefill_step(qb[a], kb[a], vb[a], pos[a], table, slots[a], cache,
                                            row, 250),), caches=(cache,))
    lib.prefill_step(qb[a], kb[a], vb[a], pos[a], table, slots[a], cache, row, 250)
    torch.cuda.synchronize()
    _replay_check("prefill_step chunk with history",
                  lambda: (lib.prefill_step(qb[b], kb[b], vb[b], pos[b], table, slots[b], cache,
                                            row, 400),), caches=(cache,))
