"""Helpers for the GPU parity tests: the same seeded inputs go to the HIP library (through
its binding) and to the CPU oracle; nothing here computes the method itself."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
from oracle import attention, paged, quant

FILL_CODE = 0x5A          # sentinel in untouched cache bytes
FILL_SCALE = -1.0         # sentinel in untouched scale slots


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return up(bits.view(np.int16)).view(torch.bfloat16)


def gpu_cache(num_pages: int, n_kv_heads: int) -> lib.PagedCache:
    c = lib.alloc_cache(num_pages, n_kv_heads)
    c.k_cache.fill_(FILL_CODE); c.v_cache.fill_(FILL_CODE)
    c.k_scale.fill_(FILL_SCALE); c.v_scale.fill_(FILL_SCALE)
    return c


def oracle_cache(num_pages: int, n_kv_heads: int):
    return paged.alloc_cache(num_pages, n_kv_heads, FILL_CODE, FILL_SCALE)


def cache_to_host(c: lib.PagedCache):
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (c.k_cache, c.v_cache, c.k_scale, c.v_scale))


class DecodeSetup:
    """A DecodeCase written into a GPU cache with kv_quant_write, plus the oracle's
    logical codes of every sequence (kept only for the sequences asked for)."""

    def __init__(self, case, keep=None, threads=8):
        self.case = case
        H = case.n_kv_heads
        self.cache = gpu_cache(case.num_pages, H)
        keep = set(range(case.num_seqs)) if keep is None else set(keep)
        self.ref = {}
        nq = case.q_rows_per_seq
        self.q_rows = np.zeros((case.num_seqs, nq, case.n_q_heads, case.head_dim), np.uint16)
        self.vmax = 0.0

        def gen(s):
            return s, case.seq_data(s), case.seq_slots(s)

        every = max(8, case.num_seqs // 8)
        with ThreadPoolExecutor(threads) as ex:
            for s, (k, v, q), slots in ex.map(gen, range(case.num_seqs)):
                if s % every == every - 1:
                    say(f"    generated and written {s + 1}/{case.num_seqs} sequences")
                lib.kv_quant_write(up(k), up(v), up(slots), self.cache)
                vc, vs = quant.quantize_rows(v)
                self.vmax = max(self.vmax, float(np.max(np.abs(quant.dequantize(vc, vs)))))
                self.q_rows[s] = q
                if s in keep:
                    kc, ks = quant.quantize_rows(k)
                    self.ref[s] = (kc, ks, vc, vs)
        torch.cuda.synchronize()
        self.q_bits = self.q_rows[:, 0]
        self.q = bf16_tensor(self.q_bits)          # first query row of each sequence
        self.q_all = bf16_tensor(self.q_rows)      # [S, nq, Hq, D]
        self.table = up(case.block_table)
        self.ctx = up(case.context_lens)

    def oracle_out(self, s, sm_scale=1.0 / 16):
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(self.q_bits[s]))
        return attention.decode_exact(qc, qs, self.ref[s], sm_scale)

    def run(self, **kw):
        out = lib.attn_decode(self.q, self.cache, self.table, self.ctx,
                              int(self.case.max_context_len), **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def oracle_verify(self, s, sm_scale=1.0 / 16):
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(self.q_rows[s]))
        return attention.verify_exact(qc, qs, self.ref[s], sm_scale)

    def oracle_int8p(self, s, sm_scale=1.0 / 16):
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(self.q_rows[s]))
        return attention.verify_int8p(qc, qs, self.ref[s], sm_scale)

    def run_int8p(self, **kw):
        out = lib.attn_decode_int8p(self.q_all, self.cache, self.table, self.ctx,
                                    int(self.case.max_context_len), **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def run_verify(self, **kw):
        out = lib.attn_verify(self.q_all, self.cache, self.table, self.ctx,
                              int(self.case.max_context_len), **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()


class PrefillSetup:
    def __init__(self, case):
        self.case = case
        k, v, q, slots = case.data()
        self.cache = gpu_cache(case.num_pages, case.n_kv_heads)
        lib.kv_quant_write(up(k), up(v), up(slots), self.cache)
        self.kc, self.ks = quant.quantize_rows(k)
        self.vc, self.vs = quant.quantize_rows(v)
        self.vmax = float(np.max(np.abs(quant.dequantize(self.vc, self.vs))))
        self.q_bits = q
        self.q = bf16_tensor(q)
        self.table = up(case.block_table)
        torch.cuda.synchronize()

    def run(self, causal=True):
        out = lib.attn_prefill_chunk(self.q, self.cache, self.table, self.case.context_len, causal)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def last_key(self, rows, causal=True):
        c = self.case
        rows = np.asarray(rows)
        return (c.context_len - c.n_new + rows) if causal else np.full(rows.shape, c.context_len - 1)

    def oracle(self, rows, causal=True, int8p=False, sm_scale=1.0 / 16):
        rows = np.asarray(rows)
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(self.q_bits[rows]))
        qd = quant.dequantize(qc, qs)
        kd = quant.dequantize(self.kc, self.ks)
        last = self.last_key(rows, causal)
        if int8p:
            return attention.attention_int8p(qd, kd, self.vc, self.vs, sm_scale, last)
        return attention.attention_exact(qd, kd, quant.dequantize(self.vc, self.vs), sm_scale, last)
