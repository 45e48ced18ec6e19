"""Pins of the oracle's attention functions against brute force, closed forms and
invariants (gfx936 INT8 KV article §1.3, §3.3; dot4-flash-attention README online
softmax and split-K; strata PR #3381 FP64 host reference and cross-kernel check)."""
import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle import paged, quant

SM = 1.0 / 16.0


def _rand(seed, R, Hq, N, Hkv, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((R, Hq, D)), rng.standard_normal((N, Hkv, D)),
            rng.standard_normal((N, Hkv, D)))


@pytest.mark.parametrize("D,Hq,Hkv,N", [(8, 6, 2, 13), (16, 4, 1, 40), (8, 3, 3, 1)])
def test_exact_matches_brute_force(D, Hq, Hkv, N):
    q, k, v = _rand(D + N, 3, Hq, N, Hkv, D)
    last = np.array([N - 1, max(0, N - 3), 0])
    sm = 1.0 / np.sqrt(D)
    ref = A.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), sm, last)
    out = A.attention_exact(q, k, v, sm, last)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_gqa_uses_contiguous_groups():
    q, k, v = _rand(3, 1, 6, 20, 2, 8)
    v[:, 1, :] += 100.0          # KV head 1 is far from head 0
    out = A.attention_exact(q, k, v, SM, [19])
    assert np.all(out[0, :3] < 50) and np.all(out[0, 3:] > 50)


def test_weights_sum_to_one():
    q, k, _ = _rand(4, 2, 6, 77, 2, 16)
    out = A.attention_exact(q, k, np.ones((77, 2, 16)), SM, [76, 30])
    assert np.max(np.abs(out - 1.0)) <= 1e-13


def test_ctx1_returns_v_exactly():
    q, k, v = _rand(5, 1, 6, 1, 2, 16)
    out = A.attention_exact(q, k, v, SM, [0])
    assert np.array_equal(out[0, :3], np.broadcast_to(v[0, 0], (3, 16)))
    assert np.array_equal(out[0, 3:], np.broadcast_to(v[0, 1], (3, 16)))


def test_zero_query_and_equal_keys_give_mean():
    _, k, v = _rand(6, 1, 6, 50, 2, 16)
    out = A.attention_exact(np.zeros((1, 6, 16)), k, v, SM, [29])
    assert np.max(np.abs(out[0, 0] - v[:30, 0].mean(0))) <= 1e-13
    q, _, _ = _rand(7, 1, 6, 1, 2, 16)
    keq = np.broadcast_to(k[:1], k.shape)
    out = A.attention_exact(q, keq, v, SM, [49])
    assert np.max(np.abs(out[0, 4] - v[:, 1].mean(0))) <= 1e-13


def test_dominant_key():
    q, k, v = _rand(8, 1, 6, 40, 2, 16)
    k[17] = q[0, 0] * 2000.0      # head 0's score on key 17 is far above the rest
    out = A.attention_exact(q, k, v, SM, [39])
    assert np.max(np.abs(out[0, 0] - v[17, 0])) <= 1e-12


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(9)
    ctx = 1300                   # partitions 512, 512, 276
    q = rng.standard_normal((24, 256)); k = rng.standard_normal((ctx, 4, 256))
    v = rng.standard_normal((ctx, 4, 256)) * 3
    m, l, o = A.split_partials(q, k, v, SM, ctx)
    assert m.shape == (24, 3)
    merged = A.merge_partials(m, l, o)
    exact = A.attention_exact(q[None], k, v, SM, [ctx - 1])[0]
    assert np.max(np.abs(merged - exact)) <= 1e-12 * np.abs(exact).max()


def _quantized_case(seed, ctx_lens, pages):
    case = workloads.make_decode_case(seed, ctx_lens, pages=pages, k_outliers=4)
    k, v, q, slots = case.all_data()
    kc, ks = quant.quantize_rows(k); vc, vs = quant.quantize_rows(v)
    qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q))
    cache = paged.alloc_cache(case.num_pages, 4)
    paged.write_rows(cache, slots, kc, ks, vc, vs)
    return case, cache, qc, qs


def test_page_permutation_invariance():
    c1, cache1, qc1, qs1 = _quantized_case(31, [200], "identity")
    c2, cache2, qc2, qs2 = _quantized_case(31, [200], "random")
    assert not np.array_equal(c1.block_table, c2.block_table)
    o1 = A.decode_exact(qc1[0, 0], qs1[0, 0], paged.gather_seq(cache1, c1.block_table[0], 200, 4), SM)
    o2 = A.decode_exact(qc2[0, 0], qs2[0, 0], paged.gather_seq(cache2, c2.block_table[0], 200, 4), SM)
    assert np.array_equal(o1, o2)


def test_chunk_row_equals_decode_at_matching_context():
    rng = np.random.default_rng(10)
    ctx, n_new = 90, 20
    q = rng.standard_normal((n_new, 6, 16)); k = rng.standard_normal((ctx, 2, 16))
    v = rng.standard_normal((ctx, 2, 16))
    last = ctx - n_new + np.arange(n_new)
    chunk = A.attention_exact(q, k, v, SM, last)
    for t in (0, 7, 19):
        c2 = ctx - n_new + t + 1
        dec = A.attention_exact(q[t:t + 1], k[:c2], v[:c2], SM, [c2 - 1])
        assert np.max(np.abs(chunk[t] - dec[0])) <= 1e-13


# ---- multi-row decode (verify) ----

def _verify_case(seed, ctx, nq):
    case = workloads.make_decode_case(seed, [ctx], pages="random", k_outliers=4, q_rows_per_seq=nq)
    k, v, q, slots = case.all_data()
    kc, ks = quant.quantize_rows(k); vc, vs = quant.quantize_rows(v)
    qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q[0]))
    cache = paged.alloc_cache(case.num_pages, 4)
    paged.write_rows(cache, slots, kc, ks, vc, vs)
    return paged.gather_seq(cache, case.block_table[0], ctx, 4), qc, qs


def test_verify_rows_equal_decode_at_their_own_context():
    view, qc, qs = _verify_case(41, 37, 4)          # rows at positions 33..36, across a page edge
    out = A.verify_exact(qc, qs, view, SM)
    for i in range(4):
        c_i = 37 - 4 + i + 1
        trunc = tuple(a[:c_i] for a in view)
        dec = A.decode_exact(qc[i], qs[i], trunc, SM)
        assert np.max(np.abs(out[i] - dec)) <= 1e-13   # summation order only
    assert not np.allclose(out[0], out[3])


def test_verify_one_row_is_decode():
    view, qc, qs = _verify_case(42, 50, 1)
    assert np.array_equal(A.verify_exact(qc, qs, view, SM)[0], A.decode_exact(qc[0], qs[0], view, SM))


def test_verify_matches_brute_force_tiny():
    rng = np.random.default_rng(43)
    N, nq, Hkv, Hq, D = 7, 3, 1, 2, 8
    kc = rng.integers(-127, 128, (N, Hkv, D)).astype(np.int8); ks = rng.uniform(0.01, 0.03, (N, Hkv))
    vc = rng.integers(-127, 128, (N, Hkv, D)).astype(np.int8); vs = rng.uniform(0.01, 0.03, (N, Hkv))
    qc = rng.integers(-127, 128, (nq, Hq, D)).astype(np.int8); qs = rng.uniform(0.01, 0.03, (nq, Hq))
    out = A.verify_exact(qc, qs, (kc, ks, vc, vs), 0.35)
    ref = A.brute_force_attention(quant.dequantize(qc, qs).tolist(), quant.dequantize(kc, ks).tolist(),
                                  quant.dequantize(vc, vs).tolist(), 0.35, [4, 5, 6])
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_verify_rows_before_the_context_are_zero():
    rng = np.random.default_rng(44)
    kc = rng.integers(-127, 128, (2, 1, 8)).astype(np.int8); ks = np.array([[0.02], [0.03]])
    vc = rng.integers(-127, 128, (2, 1, 8)).astype(np.int8); vs = np.array([[0.05], [0.07]])
    qc = rng.integers(-127, 128, (4, 6, 8)).astype(np.int8); qs = np.full((4, 6), 0.02)
    out = A.verify_exact(qc, qs, (kc, ks, vc, vs), SM)   # rows at positions -2, -1, 0, 1
    assert np.all(out[:2] == 0.0)
    vdeq = quant.dequantize(vc, vs)
    assert np.array_equal(out[2], np.broadcast_to(vdeq[0, 0], (6, 8)))   # one key: V itself


def test_verify_int8p_rows_equal_int8p_at_their_own_context():
    view, qc, qs = _verify_case(45, 150, 3)         # rows at 147..149: the third 64-key block
    out = A.verify_int8p(qc, qs, view, SM)
    kc, ks, vc, vs = view
    for i in range(3):
        c_i = 150 - 3 + i + 1
        ref = A.attention_int8p(quant.dequantize(qc[i:i + 1], qs[i:i + 1]),
                                quant.dequantize(kc[:c_i], ks[:c_i]), vc[:c_i], vs[:c_i], SM,
                                [c_i - 1])[0]
        assert np.max(np.abs(out[i] - ref)) <= 1e-13


def test_verify_int8p_matches_brute_force_tiny():
    rng = np.random.default_rng(46)
    N, nq, D = 70, 2, 8                               # crosses one 64-key block edge
    kc = rng.integers(-127, 128, (N, 1, D)).astype(np.int8); ks = rng.uniform(0.01, 0.03, (N, 1))
    vc = rng.integers(-127, 128, (N, 1, D)).astype(np.int8); vs = rng.uniform(0.01, 0.03, (N, 1))
    qc = rng.integers(-127, 128, (nq, 2, D)).astype(np.int8); qs = rng.uniform(0.01, 0.03, (nq, 2))
    out = A.verify_int8p(qc, qs, (kc, ks, vc, vs), 0.35)
    ref = A.brute_force_int8p(quant.dequantize(qc, qs).tolist(), quant.dequantize(kc, ks).tolist(),
                              vc.tolist(), vs.tolist(), 0.35, [N - 2, N - 1])
    assert np.max(np.abs(out - ref)) <= 1e-12


# ---- int8-P emulation (oracle B) ----

def test_int8p_matches_brute_force():
    rng = np.random.default_rng(12)
    N = 23
    q = rng.standard_normal((2, 4, 8)); k = rng.standard_normal((N, 2, 8))
    vc = rng.integers(-127, 128, (N, 2, 8)).astype(np.int8)
    vs = rng.uniform(0.01, 0.05, (N, 2)).astype(np.float32)
    last = np.array([N - 1, 9])
    ref = A.brute_force_int8p(q.tolist(), k.tolist(), vc.tolist(), vs.tolist(), SM, last, block=4)
    out = A.attention_int8p(q, k, vc, vs, SM, last, block=4)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_int8p_hand_worked_two_blocks():
    """A case worked by hand. One query, 4 keys, blocks of 2, scores 0, -ln 4, -ln 2,
    -ln 8 (sm_scale 1), so p = 1, 1/4, 1/2, 1/8 and l = 15/8; V scales 1, 1, 2, 5 and V
    codes 2, -3, 5, 7. Weights w = p * sV: block 0 (1, 1/4), s_b = 1/127, codes 127 and
    rint(31.75) = 32; block 1 (1, 5/8), s_b = 1/127, codes 127 and rint(79.375) = 79.
    Output = ((127*2 - 32*3) + (127*5 + 79*7)) / 127 / (15/8) = 1346 / 238.125.
    (Quantizing p before the V scale is folded in would give 1353 / 238.125; exact
    attention gives 10.625 / 1.875.)"""
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[-np.log(4.0)]], [[-np.log(2.0)]], [[-np.log(8.0)]]])
    vc = np.array([[[2]], [[-3]], [[5]], [[7]]], dtype=np.int8)
    vs = np.array([[1.0], [1.0], [2.0], [5.0]], np.float32)
    out = A.attention_int8p(q, k, vc, vs, 1.0, [3], block=2)
    assert abs(out[0, 0, 0] - 1346 / 238.125) <= 1e-12
    exact = A.attention_exact(q, k, quant.dequantize(vc, vs), 1.0, [3])
    assert abs(exact[0, 0, 0] - 10.625 / 1.875) <= 1e-12


def test_int8p_exact_when_block_weights_equal():
    rng = np.random.default_rng(13)
    N = 130
    k = rng.standard_normal((N, 2, 16))
    vc = rng.integers(-127, 128, (N, 2, 16)).astype(np.int8)
    vs = np.full((N, 2), 0.03, np.float32)
    q = np.zeros((1, 6, 16))   # equal scores -> equal p -> all codes 127
    outB = A.attention_int8p(q, k, vc, vs, SM, [N - 1])
    outA = A.attention_exact(q, k, quant.dequantize(vc, vs), SM, [N - 1])
    assert np.max(np.abs(outB - outA)) <= 1e-14


def test_int8p_within_rounding_bound():
    rng = np.random.default_rng(14)
    N = 300
    q = rng.standard_normal((3, 6, 32)) * 2; k = rng.standard_normal((N, 2, 32))
    vc = rng.integers(-127, 128, (N, 2, 32)).astype(np.int8)
    vs = rng.uniform(0.01, 0.05, (N, 2)).astype(np.float32)
    last = np.array([N - 1, 150, 64])
    outB = A.attention_int8p(q, k, vc, vs, SM, last)
    outA, m, l = A.attention_exact(q, k, quant.dequantize(vc, vs), SM, last, return_stats=True)
    # |c*s_b - w| <= s_b/2 per key, so |B - A| <= sum_b (s_b/2) sum_k |vcode_k| / l.
    s = np.einsum("rhd,nhd->rhn", q, np.repeat(k, 3, axis=1)) * SM
    for r in range(3):
        for h in range(6):
            g = h // 3
            n = last[r] + 1
            w = np.exp(s[r, h, :n] - m[r, h]) * vs[:n, g]
            bound = 0.0
            for b0 in range(0, n, 64):
                sb = w[b0:b0 + 64].max() / 127
                bound += sb / 2 * np.abs(vc[b0:min(n, b0 + 64), g].astype(np.float64)).sum(0)
            assert np.all(np.abs(outB[r, h] - outA[r, h]) <= bound / l[r, h] + 1e-15)
    assert np.max(np.abs(outB - outA)) > 0
