"""Whole-configuration parity for the two largest workloads: every query row of the
config-4 prefill chunk and every sequence of the config-5 batched decode, against the
oracle (exact attention, and the int8-P rule), plus config 5's cache codes and scales
bit for bit. ("#3381 prompt QSA attention without the decode kernel's split and merge",
Validation: the whole synthetic problem against an FP64 host reference; "INT8 KV and
INT8 MMAC attention on a gfx936 DCU" §2.1 codes and scales, §3.3 decode, §3.2 chunk.)

The oracle runs on row chunks (config 4) or sequences (config 5) in a thread pool with
one BLAS thread per worker; rows and sequences are independent in its definition, so
the split changes nothing in what it computes. Config 5 is streamed: each sequence is
generated, quantized by the oracle, written to the GPU cache, checked bit for bit and
reduced to its oracle outputs before the next wave of sequences, so the host never holds
the whole batch's fp32 rows (about 14 GB)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from oracle import attention, paged, quant
from tests.gpu_support import (FILL_CODE, FILL_SCALE, PrefillSetup, bf16_tensor, gpu_cache,
                               need_gpu, say, up)

pytestmark = pytest.mark.gpu

TOL_EXACT_FP32P = 1e-4   # fp32-class weights (attn_decode)
TOL_A = 1e-2             # int8 weights vs exact attention
TOL_B = 1e-3             # int8 weights vs the int8-P rule (diagnostic bar)


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


@pytest.mark.timeout(900)
def test_config4_every_row_both_oracles():
    need_gpu()
    case = workloads.config_case(4)
    say(f"attn_prefill_chunk config 4: all {case.n_new} rows x {case.n_q_heads} heads at ctx "
        f"{case.context_len}")
    st = PrefillSetup(case)
    out = st.run()
    assert np.all(np.isfinite(out))
    qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(st.q_bits))
    qd = quant.dequantize(qc, qs)
    kd = quant.dequantize(st.kc, st.ks)
    vd = quant.dequantize(st.vc, st.vs)
    last = st.last_key(np.arange(case.n_new))
    chunks = [np.arange(r0, min(case.n_new, r0 + 64)) for r0 in range(0, case.n_new, 64)]

    def ref(rows):
        a = attention.attention_exact(qd[rows], kd, vd, workloads.SM_SCALE, last[rows])
        b = attention.attention_int8p(qd[rows], kd, st.vc, st.vs, workloads.SM_SCALE, last[rows])
        return rows, float(np.max(np.abs(out[rows] - a))), float(np.max(np.abs(out[rows] - b)))

    wa = wb = 0.0
    done = 0
    with _one_blas_thread(), ThreadPoolExecutor(_workers()) as ex:
        for rows, ea, eb in ex.map(ref, chunks):
            wa, wb = max(wa, ea), max(wb, eb)
            done += len(rows)
            if done % 512 == 0:
                say(f"  oracle rows {done}/{case.n_new}: worst err vs exact {wa:.3e}, "
                    f"vs int8-P rule {wb:.3e}")
    say(f"  config 4, all rows: worst abs err vs exact {wa:.3e} (bound {TOL_A * st.vmax:.3e}), "
        f"vs int8-P rule {wb:.3e} (bound {TOL_B * st.vmax:.3e}); max|V_deq| {st.vmax:.4f}")
    assert wa <= TOL_A * st.vmax
    assert wb <= TOL_B * st.vmax


class Config5:
    """Config 5 written to a GPU cache one wave of sequences at a time; keeps per sequence
    only the oracle outputs (exact decode, and the int8-P rule) and whether its pages
    matched the oracle's codes and scales byte for byte."""

    def __init__(self):
        c = workloads.config_case(5)
        self.case = c
        H = c.n_kv_heads
        self.cache = gpu_cache(c.num_pages, H)
        self.ref_a = {}
        self.ref_b = {}
        self.q = np.zeros((c.num_seqs, c.n_q_heads, c.head_dim), np.uint16)
        self.vmax = 0.0
        self.pages_checked = 0

        def work(s):
            k, v, q = c.seq_data(s)
            kc, ks = quant.quantize_rows(k)
            vc, vs = quant.quantize_rows(v)
            qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q))
            view = (kc, ks, vc, vs)
            a = attention.decode_exact(qc[0], qs[0], view, workloads.SM_SCALE)
            b = attention.verify_int8p(qc, qs, view, workloads.SM_SCALE)[0]
            vmax = float(np.max(np.abs(quant.dequantize(vc, vs))))
            return s, k, v, q[0], view, a, b, vmax

        n_w = _workers()
        order = list(range(c.num_seqs))
        with _one_blas_thread(), ThreadPoolExecutor(n_w) as ex:
            for w0 in range(0, len(order), n_w):
                for s, k, v, q, view, a, b, vmax in ex.map(work, order[w0:w0 + n_w]):
                    lib.kv_quant_write(up(k), up(v), up(c.seq_slots(s)), self.cache)
                    self._check_pages(s, view)
                    self.ref_a[s], self.ref_b[s], self.q[s] = a, b, q
                    self.vmax = max(self.vmax, vmax)
                say(f"    config 5: {min(w0 + n_w, len(order))}/{c.num_seqs} sequences written, "
                    f"checked and reduced")
        self.q_t = bf16_tensor(self.q)
        self.table = up(c.block_table)
        self.ctx = up(c.context_lens)

    def _check_pages(self, s, view):
        """The sequence's pages, as the GPU wrote them, equal the oracle's write of the
        same codes into sentinel-filled pages (so untouched slots of its last page must
        keep the sentinel)."""
        c = self.case
        H = c.n_kv_heads
        ctx = int(c.context_lens[s])
        n_pg = -(-ctx // workloads.PAGE)
        pages = torch.as_tensor(c.block_table[s, :n_pg].astype(np.int64), device="cuda")
        blk = self.cache.k_cache.view(c.num_pages, -1)
        got = [blk.index_select(0, pages).cpu().numpy().reshape(-1),
               self.cache.v_cache.view(c.num_pages, -1).index_select(0, pages).cpu().numpy().reshape(-1),
               self.cache.k_scale.view(c.num_pages, -1).index_select(0, pages).cpu().numpy().reshape(-1),
               self.cache.v_scale.view(c.num_pages, -1).index_select(0, pages).cpu().numpy().reshape(-1)]
        want = paged.alloc_cache(n_pg, H, FILL_CODE, FILL_SCALE)
        kc, ks, vc, vs = view
        paged.write_rows(want, np.arange(ctx), kc, ks, vc, vs)   # pages renumbered 0..n_pg-1
        for g, w, what in zip(got, want, ("k codes", "v codes", "k scales", "v scales")):
            assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), (s, what)
        self.pages_checked += n_pg


@pytest.fixture(scope="module")
def config5():
    need_gpu()
    c = workloads.config_case(5)
    say(f"config 5: {c.num_seqs} sequences, {c.total_tokens} tokens, {c.num_pages} pages "
        f"(contexts {int(c.context_lens.min())}..{int(c.context_lens.max())})")
    return Config5()


@pytest.mark.timeout(900)
def test_config5_cache_codes_bit_exact(config5):
    # (the comparison itself runs while the fixture streams the sequences in)
    c = config5.case
    assert config5.pages_checked == c.num_pages
    say(f"  config 5: all {c.num_pages} pages of K/V codes and scales equal the oracle's")


@pytest.mark.timeout(900)
def test_config5_decode_every_sequence(config5):
    c = config5.case
    out = lib.attn_decode(config5.q_t, config5.cache, config5.table, config5.ctx,
                          c.max_context_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    errs = [float(np.max(np.abs(out[s] - config5.ref_a[s]))) for s in range(c.num_seqs)]
    worst = int(np.argmax(errs))
    say(f"  config 5 attn_decode, all {c.num_seqs} sequences: worst abs err {errs[worst]:.3e} "
        f"(sequence {worst}, ctx {int(c.context_lens[worst])}; bound "
        f"{TOL_EXACT_FP32P * config5.vmax:.3e})")
    assert max(errs) <= TOL_EXACT_FP32P * config5.vmax


@pytest.mark.timeout(900)
def test_config5_int8p_decode_every_sequence(config5):
    c = config5.case
    out = lib.attn_decode_int8p(config5.q_t, config5.cache, config5.table, config5.ctx,
                                c.max_context_len)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ea = [float(np.max(np.abs(out[s] - config5.ref_a[s]))) for s in range(c.num_seqs)]
    eb = [float(np.max(np.abs(out[s] - config5.ref_b[s]))) for s in range(c.num_seqs)]
    say(f"  config 5 attn_decode_int8p, all {c.num_seqs} sequences: worst err vs exact "
        f"{max(ea):.3e} (bound {TOL_A * config5.vmax:.3e}), vs int8-P rule {max(eb):.3e} "
        f"(bound {TOL_B * config5.vmax:.3e})")
    assert max(ea) <= TOL_A * config5.vmax
    assert max(eb) <= TOL_B * config5.vmax
