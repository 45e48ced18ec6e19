"""Pins of the oracle's RoPE and fused producer ("INT8 KV and INT8 MMAC attention on a
gfx936 DCU" §2.2: RoPE, absmax, scale, quantize and paged write in one producer)."""
import numpy as np

import workloads
from oracle import paged, quant, rope


def _rows(seed, R, D=256):
    return np.random.default_rng(seed).standard_normal((R, D)).astype(np.float32)


def test_zero_angle_is_identity():
    x = _rows(1, 5)
    table = workloads.rope_table(10, 256)
    assert np.array_equal(rope.rope_rows(x, np.zeros(5, int), table, 256), x)


def test_quarter_turn_is_exact():
    x = _rows(2, 3, 16)
    table = np.concatenate([np.zeros((1, 8)), np.ones((1, 8))], axis=1).astype(np.float32)
    out = rope.rope_rows(x, np.zeros(3, int), table, 16)
    assert np.array_equal(out[:, :8], -x[:, 8:]) and np.array_equal(out[:, 8:], x[:, :8])


def test_matches_complex_multiplication():
    """Pair (x_i, x_{i+rd/2}) as the complex number x_i + i x_{i+rd/2}, times e^{i angle}."""
    x = _rows(3, 7)
    pos = np.array([0, 1, 5, 100, 4095, 77, 3])
    table = workloads.rope_table(4096, 128)
    out = rope.rope_rows(x, pos, table, 128)
    z = x[:, :64].astype(np.float64) + 1j * x[:, 64:128].astype(np.float64)
    rot = table[pos, :64].astype(np.float64) + 1j * table[pos, 64:].astype(np.float64)
    ref = z * rot
    bound = 2.0 ** -23 * (np.abs(x[:, :64]) + np.abs(x[:, 64:128])) * 2
    assert np.all(np.abs(out[:, :64] - ref.real) <= bound)
    assert np.all(np.abs(out[:, 64:128] - ref.imag) <= bound)
    assert np.array_equal(out[:, 128:], x[:, 128:])          # dims past rotary_dim pass through


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((2, 256)).astype(np.float32)
    table = workloads.rope_table(9000, 256)
    def score(m, n):
        return float(np.dot(rope.rope_rows(q, np.array(m), table, 256).astype(np.float64),
                            rope.rope_rows(k, np.array(n), table, 256).astype(np.float64)))
    base = score(40, 13)
    for d in (1, 500, 8000):
        assert abs(score(40 + d, 13 + d) - base) <= 1e-3 * (1 + abs(base))
    assert abs(score(41, 13) - base) > 1e-2                   # and on nothing less


def test_producer_is_rope_then_quantize_then_write():
    case = workloads.make_producer_case(5, 40, start=7)
    q, k, v = case.data()
    table = case.table()
    cache = paged.alloc_cache(case.num_pages, 4, 0, 0.0)
    qc, qs = rope.produce(q, k, v, case.positions, table, 256, case.slots, cache)
    pos = case.positions.astype(np.int64)
    kc, ks = quant.quantize_rows(rope.rope_rows(k, pos[:, None], table, 256))
    vc, vs = quant.quantize_rows(v)
    for t in (0, 8, 39):
        p, o = divmod(int(case.slots[t]), 16)
        kk = cache[0][paged.k_offset(p, np.arange(4)[:, None], o, np.arange(256)[None, :], 4)]
        vv = cache[1][paged.v_offset(p, np.arange(4)[:, None], o, np.arange(256)[None, :], 4)]
        assert np.array_equal(kk, kc[t]) and np.array_equal(vv, vc[t])
        assert np.array_equal(cache[2][paged.scale_index(p, np.arange(4), o, 4)], ks[t])
    # Q codes are the quantized rotated rows; dequantized they sit within half a code of them
    qr = rope.rope_rows(q, pos[:, None], table, 256)
    assert np.all(np.abs(quant.dequantize(qc, qs) - qr) <= 0.5001 * qs[..., None])


def test_first_chunk_producer_writes_the_same_cache_and_rounds_the_rotated_rows():
    case = workloads.make_producer_case(6, 33, start=0)
    q, k, v = case.data()
    table = case.table()
    c1 = paged.alloc_cache(case.num_pages, 4, 0, 0.0)
    c2 = paged.alloc_cache(case.num_pages, 4, 0, 0.0)
    rope.produce(q, k, v, case.positions, table, 256, case.slots, c1)
    qb, kb = rope.produce_first_chunk(q, k, v, case.positions, table, 256, case.slots, c2)
    for a, b in zip(c1, c2):
        assert np.array_equal(a, b)
    pos = case.positions.astype(np.int64)[:, None]
    qr = rope.rope_rows(q, pos, table, 256)
    back = quant.bf16_bits_to_f32(qb)
    # nearest bf16: within half a bf16 ulp (at most 2^-8 relative) of the fp32 value
    assert np.all(np.abs(back - qr) <= np.abs(qr) * 2.0 ** -8)
    assert np.array_equal(kb, quant.f32_to_bf16_rne(rope.rope_rows(k, pos, table, 256)))
