"""A softmax scale of 0 (the calls accept any finite sm_scale >= 0) weights every visible
key alike: each attention route must return the mean of the visible V rows. Checked
against the oracle run with the same scale 0, at each route's own bound (decode, verify
and the bf16 chunk 1e-4 * max|V|; the int8 chunk 1e-2 vs exact and 1e-3 vs the int8-P
emulation; the int8-P decode 1e-2). The int8 and bf16 chunk kernels run a scale of 0 as
1e-30, which must give the same weights in fp32."""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from oracle import attention, quant
from tests.gpu_support import DecodeSetup, PrefillSetup, bf16_tensor, need_gpu, say

pytestmark = pytest.mark.gpu


def test_zero_scale_decode_verify_int8p():
    need_gpu()
    ctx = [1, 100, 700, 3000]
    say(f"sm_scale = 0: attn_decode, attn_verify (nq = 4), attn_decode_int8p over contexts {ctx}")
    case = workloads.make_decode_case(91, ctx, pages="random", k_outliers=4, extra_pages=2,
                                      q_rows_per_seq=4)
    st = DecodeSetup(case)
    dec = st.run(sm_scale=0.0)
    ver = st.run_verify(sm_scale=0.0)
    i8p = st.run_int8p(sm_scale=0.0)
    worst = [0.0, 0.0, 0.0]
    for s in range(len(ctx)):
        kc, ks, vc, vs = st.ref[s]
        mean = quant.dequantize(vc, vs).mean(axis=0)          # [Hkv, D]: the uniform weights
        e_dec = float(np.max(np.abs(dec[s] - st.oracle_out(s, sm_scale=0.0))))
        e_ver = float(np.max(np.abs(ver[s] - st.oracle_verify(s, sm_scale=0.0))))
        e_i8p = float(np.max(np.abs(i8p[s] - st.oracle_int8p(s, sm_scale=0.0))))
        # the oracle's rows are the plain means: row h of a query sees KV head h // 6
        ref = st.oracle_out(s, sm_scale=0.0)
        assert np.allclose(ref, np.repeat(mean, 6, axis=0), rtol=0, atol=1e-12)
        worst = [max(worst[0], e_dec), max(worst[1], e_ver), max(worst[2], e_i8p)]
        assert e_dec <= 1e-4 * st.vmax, (s, e_dec)
        assert e_ver <= 1e-4 * st.vmax, (s, e_ver)
        assert e_i8p <= 1e-2 * st.vmax, (s, e_i8p)
    say(f"  worst err decode {worst[0]:.3e}, verify {worst[1]:.3e}, int8-P {worst[2]:.3e} "
        f"(max|V| {st.vmax:.3f})")


@pytest.mark.parametrize("split", [False, True])
def test_zero_scale_prefill_chunk(split):
    need_gpu()
    ctx, n_new = 1200, 96
    say(f"sm_scale = 0: attn_prefill_chunk ctx={ctx} n_new={n_new} (split route: {split})")
    st = PrefillSetup(workloads.make_prefill_case(93, ctx, n_new, k_outliers=4, extra_pages=2))
    if split:
        out = lib.attn_prefill_chunk_split(st.q, st.cache, st.table, ctx, True, sm_scale=0.0)
    else:
        out = lib.attn_prefill_chunk(st.q, st.cache, st.table, ctx, True, sm_scale=0.0)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    rows = np.arange(n_new)
    ea = float(np.max(np.abs(o[rows] - st.oracle(rows, sm_scale=0.0))))
    eb = float(np.max(np.abs(o[rows] - st.oracle(rows, int8p=True, sm_scale=0.0))))
    say(f"  err vs exact {ea:.3e}, vs int8-P emulation {eb:.3e} (max|V| {st.vmax:.3f})")
    assert ea <= 1e-2 * st.vmax and eb <= 1e-3 * st.vmax


@pytest.mark.parametrize("split", [False, True])
def test_zero_scale_chunk_bf16(split):
    need_gpu()
    n = 700
    say(f"sm_scale = 0: attn_chunk_bf16 n={n} causal (key partitions: {split})")
    rng = np.random.default_rng(95)
    q = rng.standard_normal((n, 24, 256), dtype=np.float32)
    k = rng.standard_normal((n, 4, 256), dtype=np.float32)
    v = rng.standard_normal((n, 4, 256), dtype=np.float32)
    qb, kb, vb = (workloads.f32_to_bf16_bits(a) for a in (q, k, v))
    out = lib.attn_chunk_bf16(bf16_tensor(qb), bf16_tensor(kb), bf16_tensor(vb), causal=True,
                              sm_scale=0.0, split=split)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    qd, kd, vd = (quant.bf16_bits_to_f32(a).astype(np.float64) for a in (qb, kb, vb))
    rows = np.arange(n)
    ref = attention.attention_exact(qd, kd, vd, 0.0, rows)
    # row t: the mean of V rows 0..t of its KV head
    cm = np.cumsum(vd, axis=0) / np.arange(1, n + 1)[:, None, None]
    assert np.allclose(ref, np.repeat(cm, 6, axis=1), rtol=0, atol=1e-12)
    vmax = float(np.max(np.abs(vd)))
    err = float(np.max(np.abs(o - ref)))
    say(f"  err {err:.3e} (bound {1e-4 * vmax:.3e})")
    assert err <= 1e-4 * vmax
