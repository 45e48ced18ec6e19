"""The high-precision route of a chunk with no history ("INT8 KV and INT8 MMAC attention
on a gfx936 DCU" §3.1, §3.2): attn_chunk_bf16 against exact attention on the same bf16
rows (max abs error <= 1e-4 * max|V|, the fp32-class bar), the producer's rotated bf16
rows bit for bit, and prefill_step's routing: no history -> bf16 attention on the rotated
rows, a history -> the int8 chunk path on the producer's Q codes."""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from oracle import attention, paged, quant, rope
from tests.gpu_support import cache_to_host, gpu_cache, need_gpu, oracle_cache, say, up

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _bf16(bits):
    return up(bits.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("n,causal", [(1, True), (33, True), (64, True), (300, True),
                                      (300, False), (2048, True)])
def test_chunk_bf16_matches_exact(n, causal):
    need_gpu()
    say(f"attn_chunk_bf16 n={n} causal={causal}")
    rng = np.random.default_rng(200 + n)
    q = rng.standard_normal((n, 24, 256), dtype=np.float32)
    k = rng.standard_normal((n, 4, 256), dtype=np.float32)
    k[:, :, rng.choice(256, 4, replace=False)] *= np.float32(10.0)
    v = rng.standard_normal((n, 4, 256), dtype=np.float32)
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    out = lib.attn_chunk_bf16(_bf16(qb), _bf16(kb), _bf16(vb), causal=causal)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    qd, kd, vd = (quant.bf16_bits_to_f32(a).astype(np.float64) for a in (qb, kb, vb))
    rows = np.arange(n)   # every row, n = 2,048 included
    last = rows if causal else np.full(rows.shape, n - 1)
    ref = attention.attention_exact(qd[rows], kd, vd, 1 / 16, last)
    vmax = float(np.max(np.abs(vd)))
    err = float(np.max(np.abs(o[rows] - ref)))
    say(f"  err {err:.3e} (bound {TOL * vmax:.3e})")
    assert err <= TOL * vmax


@pytest.mark.parametrize("n,n_kv", [(300, 4), (1000, 1), (700, 3), (2048, 4)])
def test_chunk_bf16_split_equals_one_pass(n, n_kv):
    # causal chunks cut into key partitions (workspace given) against the one pass: the
    # same products and softmax, only the merge's rounding differs; the rows below the
    # first partition boundary are written by the same code path as the one pass
    need_gpu()
    ws = lib.attn_chunk_bf16_workspace_bytes(n, True, 6 * n_kv, n_kv)
    say(f"attn_chunk_bf16 n={n} with {n_kv} KV heads: split workspace {ws} B vs the one pass")
    assert ws > 0
    rng = np.random.default_rng(260 + n)
    q = rng.standard_normal((n, 6 * n_kv, 256), dtype=np.float32)
    k = rng.standard_normal((n, n_kv, 256), dtype=np.float32)
    v = rng.standard_normal((n, n_kv, 256), dtype=np.float32)
    qb, kb, vb = (_bf16(workloads.f32_to_bf16_bits(a)) for a in (q, k, v))
    wbuf = torch.full((ws,), 0xff, dtype=torch.uint8, device="cuda")  # NaN bit patterns
    a = lib.attn_chunk_bf16(qb, kb, vb, causal=True, workspace=wbuf).cpu().numpy()
    b = lib.attn_chunk_bf16(qb, kb, vb, causal=True, split=False).cpu().numpy()
    vmax = float(np.max(np.abs(v)))
    d = float(np.max(np.abs(a - b)))
    say(f"  max |split - one pass| {d:.3e} (bound {1e-5 * vmax:.3e})")
    assert np.all(np.isfinite(a)) and d <= 1e-5 * vmax
    # the first rows of every tile below the boundary are bit-identical
    assert np.array_equal(a[:64], b[:64])


@pytest.mark.parametrize("n,parted", [(3000, True), (6000, False)])
def test_chunk_bf16_long_ragged_chunk(n, parted):
    # long chunks with a ragged last block of 64 keys: at 3,000 rows the plan cuts the keys
    # into partitions; at 6,000 rows (752 workgroups for 256 CUs) it keeps the one pass.
    # 48 rows across the chunk, the last ones included, against exact attention on the
    # same bf16 rows, and the default route against the one pass on every row
    need_gpu()
    ws = lib.attn_chunk_bf16_workspace_bytes(n, True, 24, 4)
    say(f"attn_chunk_bf16 n={n} causal: split workspace {ws} B, 48 rows vs exact")
    assert (ws > 0) == parted
    rng = np.random.default_rng(270 + n)
    q = rng.standard_normal((n, 24, 256), dtype=np.float32)
    k = rng.standard_normal((n, 4, 256), dtype=np.float32)
    k[:, :, rng.choice(256, 4, replace=False)] *= np.float32(10.0)
    v = rng.standard_normal((n, 4, 256), dtype=np.float32)
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    a = lib.attn_chunk_bf16(_bf16(qb), _bf16(kb), _bf16(vb), causal=True).cpu().numpy()
    b = lib.attn_chunk_bf16(_bf16(qb), _bf16(kb), _bf16(vb), causal=True, split=False).cpu().numpy()
    qd, kd, vd = (quant.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb))
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), np.arange(n - 8, n)]))
    ref = attention.attention_exact(qd[rows], kd, vd, 1 / 16, rows)
    vmax = float(np.max(np.abs(vd)))
    err = max(float(np.max(np.abs(a[rows] - ref))), float(np.max(np.abs(b[rows] - ref))))
    d = float(np.max(np.abs(a - b)))
    say(f"  err {err:.3e} (bound {TOL * vmax:.3e}); max |split - one pass| {d:.3e} "
        f"(bound {1e-5 * vmax:.3e})")
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    assert err <= TOL * vmax and d <= 1e-5 * vmax


@pytest.mark.parametrize("n_kv", [1, 3])
def test_chunk_bf16_other_kv_head_counts(n_kv):
    need_gpu()
    n = 77
    say(f"attn_chunk_bf16 n={n} causal with {n_kv} KV heads x 6 query heads")
    rng = np.random.default_rng(230 + n_kv)
    q = rng.standard_normal((n, 6 * n_kv, 256), dtype=np.float32)
    k = rng.standard_normal((n, n_kv, 256), dtype=np.float32)
    v = rng.standard_normal((n, n_kv, 256), dtype=np.float32)
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    out = lib.attn_chunk_bf16(_bf16(qb), _bf16(kb), _bf16(vb), causal=True)
    torch.cuda.synchronize()
    qd, kd, vd = (quant.bf16_bits_to_f32(a).astype(np.float64) for a in (qb, kb, vb))
    ref = attention.attention_exact(qd, kd, vd, 1 / 16, np.arange(n))
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    vmax = float(np.max(np.abs(vd)))
    say(f"  err {err:.3e} (bound {TOL * vmax:.3e})")
    assert err <= TOL * vmax


def test_producer_rotated_rows_bit_exact():
    need_gpu()
    case = workloads.make_producer_case(210, 300, start=0, rotary_dim=128)
    q, k, v = case.data()
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    q, k, v = (quant.bf16_bits_to_f32(a) for a in (qb, kb, vb))
    table = case.table()
    say("kv_produce with rotated bf16 outputs (300 tokens, rotary_dim 128)")
    cache = gpu_cache(case.num_pages, 4)
    qr, kr = lib.kv_produce(_bf16(qb), _bf16(kb), _bf16(vb), up(case.positions), up(table),
                            up(case.slots), cache, rotated_bf16=True)
    torch.cuda.synchronize()
    ref_cache = oracle_cache(case.num_pages, 4)
    rq, rk = rope.produce_first_chunk(q, k, v, case.positions, table, 128, case.slots, ref_cache)
    assert np.array_equal(qr.cpu().view(torch.int16).numpy().view(np.uint16), rq)
    assert np.array_equal(kr.cpu().view(torch.int16).numpy().view(np.uint16), rk)
    for a, b in zip(cache_to_host(cache), ref_cache):
        assert np.array_equal(a, b)


def test_prefill_step_routes_by_history():
    need_gpu()
    say("prefill_step: 300-token first chunk (bf16 route), then 100 tokens (int8 route, key "
        "partitions), then 5 tokens (int8 route, int8-P decode kernel)")
    full = workloads.make_producer_case(220, 405, start=0, rotary_dim=256)
    q, k, v = full.data()
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    q, k, v = (quant.bf16_bits_to_f32(a) for a in (qb, kb, vb))
    table = full.table()
    cache = gpu_cache(full.num_pages, 4)
    block_row = up((full.slots[::16] // 16).astype(np.int32))
    chunks = ((0, 300), (300, 400), (400, 405))
    outs = []
    for a, b in chunks:
        sl = slice(a, b)
        outs.append(lib.prefill_step(_bf16(qb[sl]), _bf16(kb[sl]), _bf16(vb[sl]),
                                     up(full.positions[sl]), up(table), up(full.slots[sl]), cache,
                                     block_row, b))
    torch.cuda.synchronize()
    ref_cache = oracle_cache(full.num_pages, 4)
    rq, rk = rope.produce_first_chunk(q[:300], k[:300], v[:300], full.positions[:300], table, 256,
                                      full.slots[:300], ref_cache)
    # first chunk: exact attention on the rotated bf16 rows and the input V
    qd, kd = quant.bf16_bits_to_f32(rq).astype(np.float64), quant.bf16_bits_to_f32(rk).astype(np.float64)
    ref1 = attention.attention_exact(qd, kd, v[:300].astype(np.float64), 1 / 16, np.arange(300))
    vmax = float(np.max(np.abs(v)))
    e1 = float(np.max(np.abs(outs[0].cpu().numpy() - ref1)))
    say(f"  first chunk: err {e1:.3e} (bound {TOL * vmax:.3e})")
    assert e1 <= TOL * vmax
    # later chunks: the int8 path over the int8 cache with the producer's Q codes
    for (a, b), o in zip(chunks[1:], outs[1:]):
        qc, qs = rope.produce(q[a:b], k[a:b], v[a:b], full.positions[a:b], table, 256,
                              full.slots[a:b], ref_cache)
        kc, ks, vc, vs = paged.gather_seq(ref_cache, full.slots[::16] // 16, b, 4)
        qd2 = quant.dequantize(qc, qs)
        last = a + np.arange(b - a)
        ref_a = attention.attention_exact(qd2, quant.dequantize(kc, ks), quant.dequantize(vc, vs),
                                          1 / 16, last)
        ref_b = attention.attention_int8p(qd2, quant.dequantize(kc, ks), vc, vs, 1 / 16, last)
        vmax2 = float(np.max(np.abs(quant.dequantize(vc, vs))))
        o2 = o.cpu().numpy()
        ea, eb = float(np.max(np.abs(o2 - ref_a))), float(np.max(np.abs(o2 - ref_b)))
        say(f"  chunk {a}..{b}: err vs exact {ea:.3e}, vs int8-P rule {eb:.3e} (max|V| {vmax2:.3f})")
        assert ea <= 1e-2 * vmax2 and eb <= 1e-3 * vmax2
    for a_, b_ in zip(cache_to_host(cache), ref_cache):
        assert np.array_equal(a_, b_)
