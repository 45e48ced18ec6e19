"""kv_produce (RoPE on Q/K + Q/K/V quantization + paged K/V write in one launch) against
the oracle bit for bit, and the int8-query (*_q8) attention forms: given q_quant's codes
they equal the bf16 forms bit for bit, and after the producer they match the oracle on
the rotated rows. ("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §2.2 fused producer;
§3.3: the decode consumes INT8 Q and its scale.)"""
import dataclasses

import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from oracle import attention, paged, quant, rope
from tests.gpu_support import cache_to_host, gpu_cache, need_gpu, oracle_cache, say, up

pytestmark = pytest.mark.gpu


def _bits_tensor(bits):
    return up(bits.view(np.int16)).view(torch.bfloat16)


def _run(case, in_bf16):
    q, k, v = case.data()
    table = case.table()
    if in_bf16:
        qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
        q, k, v = (quant.bf16_bits_to_f32(a) for a in (qb, kb, vb))   # what the kernel sees
        tq, tk, tv = (_bits_tensor(a) for a in (qb, kb, vb))
    else:
        tq, tk, tv = up(q), up(k), up(v)
    cache = gpu_cache(case.num_pages, case.n_kv_heads)
    qc, qs = lib.kv_produce(tq, tk, tv, up(case.positions), up(table), up(case.slots), cache,
                            rotary_dim=case.rotary_dim)
    torch.cuda.synchronize()
    ref_cache = oracle_cache(case.num_pages, case.n_kv_heads)
    rqc, rqs = rope.produce(q, k, v, case.positions, table, case.rotary_dim, case.slots, ref_cache)
    return cache, (qc, qs), ref_cache, (rqc, rqs), table


@pytest.mark.parametrize("T,start,layout,rd,in_bf16", [
    (2048, 0, "chunk", 256, True),      # a prefill chunk: whole-page runs
    (100, 7, "chunk", 128, False),      # ragged first and last page, partial rotation
    (37, 0, "scatter", 64, True),       # decode tokens of 37 sequences, some slots skipped
    (50, 3, "chunk", 0, False),         # no rotation: quant-write + q_quant
])
def test_produce_bit_exact(T, start, layout, rd, in_bf16):
    need_gpu()
    say(f"kv_produce T={T} start={start} {layout} rotary_dim={rd} bf16={in_bf16}")
    case = workloads.make_producer_case(100 + T, T, start=start, layout=layout, rotary_dim=rd)
    cache, (qc, qs), ref_cache, (rqc, rqs), _ = _run(case, in_bf16)
    got = cache_to_host(cache)
    for name, a, b in zip(("k codes", "v codes", "k scales", "v scales"), got, ref_cache):
        assert np.array_equal(a, b), name
    assert np.array_equal(qc.cpu().numpy(), rqc)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), rqs.view(np.uint32))


@pytest.mark.parametrize("n_kv", [1, 2, 3])
def test_produce_other_kv_head_counts(n_kv):
    need_gpu()
    say(f"kv_produce with {n_kv} KV heads x 6 query heads, 45 tokens from position 5")
    case = dataclasses.replace(workloads.make_producer_case(130 + n_kv, 45, start=5, rotary_dim=128),
                               n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    cache, (qc, qs), ref_cache, (rqc, rqs), _ = _run(case, True)
    for name, a, b in zip(("k codes", "v codes", "k scales", "v scales"), cache_to_host(cache), ref_cache):
        assert np.array_equal(a, b), name
    assert np.array_equal(qc.cpu().numpy(), rqc)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), rqs.view(np.uint32))


def test_q8_forms_equal_bf16_forms():
    need_gpu()
    say("attn_*_q8 with q_quant codes vs the bf16 forms")
    case = workloads.make_decode_case(110, [700, 1500], pages="random", k_outliers=4,
                                      q_rows_per_seq=3)
    from tests.gpu_support import DecodeSetup
    st = DecodeSetup(case)
    q1 = st.q                                            # [S, Hq, D] bf16
    c1, s1 = lib.q_quant(q1)
    a = lib.attn_decode(q1, st.cache, st.table, st.ctx, 1500)
    b = lib.attn_decode(c1, st.cache, st.table, st.ctx, 1500, q_scales=s1)
    c3, s3 = lib.q_quant(st.q_all)
    va = lib.attn_verify(st.q_all, st.cache, st.table, st.ctx, 1500)
    vb = lib.attn_verify(c3, st.cache, st.table, st.ctx, 1500, q_scales=s3)
    ia = lib.attn_decode_int8p(st.q_all, st.cache, st.table, st.ctx, 1500)
    ib = lib.attn_decode_int8p(c3, st.cache, st.table, st.ctx, 1500, q_scales=s3)
    pf = workloads.make_prefill_case(111, 900, 90, k_outliers=4)
    from tests.gpu_support import PrefillSetup
    ps = PrefillSetup(pf)
    cp, sp = lib.q_quant(ps.q)
    pa = lib.attn_prefill_chunk(ps.q, ps.cache, ps.table, pf.context_len, True)
    pb = lib.attn_prefill_chunk(cp, ps.cache, ps.table, pf.context_len, True, q_scales=sp)
    torch.cuda.synchronize()
    for x, y in ((a, b), (va, vb), (ia, ib), (pa, pb)):
        assert torch.equal(x, y)


def test_produce_then_attend_matches_oracle():
    """A 300-token sequence produced with RoPE in two chunks (240 + 60), then the chunk
    attention and a 3-row verify read it through the int8-query forms."""
    need_gpu()
    say("kv_produce 240 + 60 tokens, then attn_prefill_chunk_q8 and attn_verify_q8")
    full = workloads.make_producer_case(120, 300, start=0, layout="chunk", rotary_dim=256)
    q, k, v = full.data()
    table = full.table()
    cache = gpu_cache(full.num_pages, 4)
    ref_cache = oracle_cache(full.num_pages, 4)
    codes, scales = [], []
    for a, b in ((0, 240), (240, 300)):
        sl = slice(a, b)
        qc, qs = lib.kv_produce(up(q[sl]), up(k[sl]), up(v[sl]), up(full.positions[sl]), up(table),
                                up(full.slots[sl]), cache)
        codes.append(qc); scales.append(qs)
        rope.produce(q[sl], k[sl], v[sl], full.positions[sl], table, 256, full.slots[sl], ref_cache)
    block_row = (full.slots[::16] // 16).astype(np.int32)
    table_t = up(block_row)
    out = lib.attn_prefill_chunk(codes[1], cache, table_t, 300, True, q_scales=scales[1])
    torch.cuda.synchronize()
    pos = full.positions.astype(np.int64)
    qr = rope.rope_rows(q, pos[:, None], table, 256)
    rqc, rqs = quant.quantize_rows(qr)
    view = paged.gather_seq(ref_cache, block_row, 300, 4)
    kc, ks, vc, vs = view
    qd = quant.dequantize(rqc[240:], rqs[240:])
    last = 240 + np.arange(60)
    ref_a = attention.attention_exact(qd, quant.dequantize(kc, ks), quant.dequantize(vc, vs), 1 / 16, last)
    ref_b = attention.attention_int8p(qd, quant.dequantize(kc, ks), vc, vs, 1 / 16, last)
    vmax = float(np.max(np.abs(quant.dequantize(vc, vs))))
    o = out.cpu().numpy()
    ea, eb = float(np.max(np.abs(o - ref_a))), float(np.max(np.abs(o - ref_b)))
    say(f"  chunk: err vs exact {ea:.3e}, vs int8-P rule {eb:.3e} (max|V| {vmax:.3f})")
    assert ea <= 1e-2 * vmax and eb <= 1e-3 * vmax
    # the last 3 tokens as verify rows (one sequence)
    ctx_t = up(np.array([300], np.int32))
    vo = lib.attn_verify(codes[1][-3:][None].contiguous(), cache, table_t[None].contiguous(), ctx_t,
                         300, q_scales=scales[1][-3:][None].contiguous())
    torch.cuda.synchronize()
    ref_v = attention.verify_exact(rqc[297:], rqs[297:], view, 1 / 16)
    ev = float(np.max(np.abs(vo.cpu().numpy()[0] - ref_v)))
    say(f"  verify nq=3: err vs exact {ev:.3e} (bound {1e-4 * vmax:.3e})")
    assert ev <= 1e-4 * vmax
