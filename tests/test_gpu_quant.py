"""kv_quant_write and q_quant against the oracle: codes and scales bit-exact, cache bytes
outside the written slots untouched ("INT8 KV and INT8 MMAC attention on a gfx936 DCU"
§2.1 rule, §2.3 paged layout)."""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from oracle import paged, quant
from tests.gpu_support import (bf16_tensor, cache_to_host, gpu_cache, need_gpu, oracle_cache,
                               say, up)

pytestmark = pytest.mark.gpu


def _write_and_compare(k, v, slots, num_pages, H, in_bf16=False):
    cache = gpu_cache(num_pages, H)
    if in_bf16:
        kt = bf16_tensor(workloads.f32_to_bf16_bits(k)); vt = bf16_tensor(workloads.f32_to_bf16_bits(v))
        k = quant.bf16_bits_to_f32(workloads.f32_to_bf16_bits(k))
        v = quant.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v))
    else:
        kt, vt = up(k), up(v)
    lib.kv_quant_write(kt, vt, up(slots.astype(np.int32)), cache)
    got = cache_to_host(cache)
    ref = oracle_cache(num_pages, H)
    kc, ks = quant.quantize_rows(k); vc, vs = quant.quantize_rows(v)
    paged.write_rows(ref, slots, kc, ks, vc, vs)
    names = ("k_cache", "v_cache", "k_scale", "v_scale")
    for name, a, b in zip(names, got, ref):
        if a.dtype == np.float32:
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
        else:
            assert np.array_equal(a, b), name


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_rows_bit_exact(cfg):
    need_gpu()
    case = workloads.config_case(cfg)
    say(f"kv_quant_write config {cfg}")
    if cfg == 4:
        k, v, _, slots = case.data()
    else:
        k, v, _, slots = case.all_data()
    _write_and_compare(k, v, slots, case.num_pages, case.n_kv_heads)


def test_near_ties_zero_rows_and_extremes():
    need_gpu()
    rows = workloads.near_tie_rows(3, 4 * 300)
    rng = np.random.default_rng(4)
    rows[:8] = 0.0                                   # amax = 0
    rows[8, :] = 0.0; rows[8, 5] = 1e-45             # scale underflows to 0
    rows[9] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-38)  # denormal-ish scale
    rows[10] = rng.standard_normal(256).astype(np.float32) * np.float32(1e30)
    k = rows.reshape(300, 4, 256)
    v = rows[::-1].copy().reshape(300, 4, 256)
    slots = rng.permutation(40 * 16)[:300].astype(np.int32)
    _write_and_compare(k, v, slots, 40, 4)


def test_bf16_input_and_skipped_slots():
    need_gpu()
    rng = np.random.default_rng(5)
    k = rng.standard_normal((70, 4, 256)).astype(np.float32) * 3
    v = rng.standard_normal((70, 4, 256)).astype(np.float32)
    slots = rng.permutation(10 * 16)[:70].astype(np.int32)
    slots[[3, 10]] = -1                               # skipped
    slots[[20]] = 10 * 16 + 5                         # past the pool: skipped
    ref_slots = slots.copy(); ref_slots[20] = -1
    cache = gpu_cache(10, 4)
    kt = bf16_tensor(workloads.f32_to_bf16_bits(k)); vt = bf16_tensor(workloads.f32_to_bf16_bits(v))
    lib.kv_quant_write(kt, vt, up(slots), cache)
    got = cache_to_host(cache)
    ref = oracle_cache(10, 4)
    kf = quant.bf16_bits_to_f32(workloads.f32_to_bf16_bits(k))
    vf = quant.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v))
    kc, ks = quant.quantize_rows(kf); vc, vs = quant.quantize_rows(vf)
    paged.write_rows(ref, ref_slots, kc, ks, vc, vs)
    for a, b in zip(got, ref):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_other_head_counts():
    need_gpu()
    rng = np.random.default_rng(6)
    for H in (1, 3, 8):
        k = rng.standard_normal((33, H, 256)).astype(np.float32)
        v = rng.standard_normal((33, H, 256)).astype(np.float32)
        slots = rng.permutation(4 * 16)[:33].astype(np.int32)
        _write_and_compare(k, v, slots, 4, H)


def test_q_quant_bit_exact():
    need_gpu()
    case = workloads.config_case(4)
    _, _, q, _ = case.data()
    q = q[:512]
    codes, scales = lib.q_quant(bf16_tensor(q))
    torch.cuda.synchronize()
    rc, rs = quant.quantize_rows(quant.bf16_bits_to_f32(q))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    ties = workloads.f32_to_bf16_bits(workloads.near_tie_rows(9, 200))
    codes, scales = lib.q_quant(bf16_tensor(ties))
    rc, rs = quant.quantize_rows(quant.bf16_bits_to_f32(ties))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("in_bf16", [False, True])
def test_page_runs_and_scattered_slots_in_one_call(in_bf16):
    # Groups of 16 tokens: a whole page in order (written as whole blocks), the same page
    # size in reverse order, a run that starts mid-page, a whole page then a skipped
    # token inside the next run, and a ragged tail; all must equal the oracle's scatter.
    need_gpu()
    rng = np.random.default_rng(91)
    runs = [np.arange(48, 64),                 # page 3, in order
            np.arange(80, 96)[::-1],           # page 5, reversed
            np.arange(104, 120),               # starts at offset 8 of page 6
            np.arange(16, 32),                 # page 1, in order
            np.r_[np.arange(128, 135), -1, np.arange(136, 144)],  # page 8 with a skipped token
            np.array([200, 7, 250])]           # ragged tail, scattered
    slots = np.concatenate(runs).astype(np.int32)
    T, H = slots.shape[0], 2
    k = rng.standard_normal((T, H, 256), dtype=np.float32) * np.float32(2.5)
    v = rng.standard_normal((T, H, 256), dtype=np.float32)
    _write_and_compare(k, v, slots, num_pages=17, H=H, in_bf16=in_bf16)


def test_scales_across_binades_bit_exact():
    # Rows whose scales span 2^-125 .. 2^120 (every binade of a normal scale, and the first
    # denormal ones just below 2^-126) with random mantissas, plus rows whose elements sit
    # on and next to half-integer multiples of the scale at each magnitude: the codes come
    # from a reciprocal multiply away from rounding ties and from the IEEE division near
    # them, and both must give the rule's codes everywhere.
    need_gpu()
    rng = np.random.default_rng(17)
    n_rows = 4 * 512
    exps = np.concatenate([np.arange(-125, 121), np.array([-127, -128, -130, -126])])
    e = exps[rng.integers(0, exps.size, n_rows)]
    amax = np.ldexp(1.0 + rng.random(n_rows), e).astype(np.float32) * np.float32(127.0)
    rows = (rng.uniform(-1.0, 1.0, (n_rows, 256)) * amax[:, None]).astype(np.float32)
    # half the rows: elements at (k + 1/2) * scale, nudged by -1, 0, +1 ulp
    half = rows[: n_rows // 2]
    sc = (amax[: n_rows // 2] / np.float32(127.0)).astype(np.float32)
    kk = rng.integers(-126, 126, half.shape).astype(np.float32)
    tie = ((kk + np.float32(0.5)) * sc[:, None]).astype(np.float32)
    nudge = rng.integers(-1, 2, half.shape)
    tie = np.where(nudge > 0, np.nextafter(tie, np.float32(np.inf)),
                   np.where(nudge < 0, np.nextafter(tie, np.float32(-np.inf)), tie)).astype(np.float32)
    keep = np.abs(tie) < amax[: n_rows // 2, None]
    half[keep] = tie[keep]
    rows[np.arange(n_rows), rng.integers(0, 256, n_rows)] = amax     # the row's amax is exact
    finite = np.isfinite(rows).all(axis=1)
    assert finite.all()
    say(f"kv_quant_write: {n_rows} rows, scale exponents {int(e.min())}..{int(e.max())}")
    k = rows.reshape(n_rows // 4, 4, 256)
    v = rows[::-1].copy().reshape(n_rows // 4, 4, 256)
    slots = rng.permutation(64 * 16)[: n_rows // 4].astype(np.int32)
    _write_and_compare(k, v, slots, 64, 4)
    # the same rows as bf16 query rows through q_quant
    qb = workloads.f32_to_bf16_bits(rows)
    codes, scales = lib.q_quant(bf16_tensor(qb.reshape(n_rows // 4, 4, 256)))
    torch.cuda.synchronize()
    rc, rs = quant.quantize_rows(quant.bf16_bits_to_f32(qb))
    assert np.array_equal(codes.cpu().numpy().reshape(n_rows, 256), rc)
    assert np.array_equal(scales.cpu().numpy().reshape(n_rows).view(np.uint32), rs.view(np.uint32))
