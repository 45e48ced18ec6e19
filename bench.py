"""Benchmark of the INT8-KV attention hot path on one MI355X.

One step = every row of the path over one batch of synthetic input:
  1. kv_quant_write of the 2048 new rows of a causal prefill chunk (fp32 K/V in);
  2. attn_prefill_chunk: 2048 queries at the tail of a 32768-key context
     (30720 cached + 2048 new), 24 q / 4 KV heads, head_dim 256, int8 P per 64-key block;
  3. kv_quant_write of one new decode token into each of `--decode-copies` caches;
  4. attn_decode at context 32768 (split-K over 64 partitions of 512 rows + merge),
     once per cache copy, back to back. The copies are identical and are read in
     rotation, so no call finds its 68 MB working set in the 256 MB Infinity Cache
     (MALL-cold); timing the calls as one group keeps event overhead out of the
     per-call figure.

Printed: one JSON line. `value` is attn_decode microseconds per call at ctx 32768
(the headline of the metric); decode HBM GB/s, prefill int8 TOPS and MFMA utilisation,
quant-write GB/s and the per-step wall time are extra fields. Per-kernel times are HIP
events on the stream the library launches on, averaged over the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import workloads

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA


def decode_bytes(ctx: int, n_q_heads: int, n_kv_heads: int, D: int) -> int:
    """Algorithmic bytes of one decode call: every K/V code and scale of the context,
    the block table, the query, the output and the context length."""
    per_token = n_kv_heads * (2 * D + 2 * 4)
    pages = -(-ctx // workloads.PAGE)
    return ctx * per_token + pages * 4 + n_q_heads * D * 2 + n_q_heads * D * 4 + 4


def prefill_ops(ctx: int, n_new: int, n_q_heads: int, D: int) -> int:
    """int8 ops of one causal chunk: visible (query, key) pairs x heads x (QK + PV) MACs x 2."""
    pos0 = ctx - n_new
    pairs = n_new * pos0 + n_new * (n_new + 1) // 2
    return pairs * n_q_heads * 4 * D


def quant_write_bytes(n_tokens: int, n_kv_heads: int, D: int) -> int:
    """fp32 K and V rows in + slot index + int8 codes and fp32 scales out."""
    return n_tokens * (2 * n_kv_heads * D * 4 + 4 + n_kv_heads * (2 * D + 8))


def recorded_traffic(kind: str):
    """HBM bytes per launch of the `kind` ("prefill" or "decode") kernels, as measured by
    the FETCH_SIZE / WRITE_SIZE counter passes summarised under profiles/ (scaled by a
    copy of known size). Returned only while the kernel sources hash as they did when the
    counters were taken; otherwise None (the figure would describe another kernel)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "hbm_traffic_prefill_decode.md")
    src = {"prefill": ["prefill.hip", "common.hpp"], "decode": ["decode.hip", "common.hpp"]}[kind]
    try:
        fields = {}
        for line in open(path):
            if ":" in line and line.strip().startswith(kind + "_"):
                key, val = line.strip().split(":", 1)
                fields[key] = val.strip()
        h = hashlib.sha256()
        for f in src:
            h.update(open(os.path.join(root, "int8_kv_cache_amd", "csrc", f), "rb").read())
        if h.hexdigest()[:16] != fields.get(kind + "_source_sha"):
            return None
        return int(fields[kind + "_traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(dec_case, dec_data, pf_case, pf_data, budget_s=20.0):
    """The oracle, unchanged, on the host: decode at ctx 32768 (whole calls) and a
    sample of prefill query rows of the same chunk; quantization excluded."""
    from oracle import attention, quant
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    k, v, q, _ = dec_data
    kc, ks = quant.quantize_rows(k); vc, vs = quant.quantize_rows(v)
    qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q[0, 0]))
    view = (kc, ks, vc, vs)
    calls, t0 = 0, time.perf_counter()
    while True:
        attention.decode_exact(qc, qs, view, workloads.SM_SCALE)
        calls += 1
        if time.perf_counter() - t0 > budget_s / 2 or calls >= 20:
            break
    dec_us = (time.perf_counter() - t0) / calls * 1e6

    k4, v4, q4, _ = pf_data
    kc4, ks4 = quant.quantize_rows(k4); vc4, vs4 = quant.quantize_rows(v4)
    kd, vd = quant.dequantize(kc4, ks4), quant.dequantize(vc4, vs4)
    pos0 = pf_case.context_len - pf_case.n_new
    rows_done, ops, t0 = 0, 0, time.perf_counter()
    rng = np.random.default_rng(0)
    while time.perf_counter() - t0 < budget_s / 2 and rows_done < pf_case.n_new:
        rows = np.sort(rng.choice(pf_case.n_new, 16, replace=False))
        qcr, qsr = quant.quantize_rows(quant.bf16_bits_to_f32(q4[rows]))
        attention.attention_exact(quant.dequantize(qcr, qsr), kd, vd, workloads.SM_SCALE,
                                  pos0 + rows)
        rows_done += len(rows)
        ops += int(np.sum(pos0 + rows + 1)) * pf_case.n_q_heads * 4 * pf_case.head_dim
    pf_tops = ops / (time.perf_counter() - t0) / 1e12
    cores = len(os.sched_getaffinity(0))
    return {
        "decode": {"value": round(dec_us, 1), "unit": "us/call", "cores": blas_threads or cores,
                   "kind": "oracle", "host_cores": cores,
                   "sample": f"{calls} full decode calls at ctx 32768 (24 q heads), from codes"},
        "prefill": {"value": round(pf_tops, 6), "unit": "TOPS (int8-equivalent ops/s)",
                    "cores": blas_threads or cores, "kind": "oracle", "host_cores": cores,
                    "sample": f"{rows_done} of 2048 query tokens (all 24 heads) of the chunk"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, one device-to-device copy of this many MiB "
                         "(reference dispatch for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build measures the single-GPU path "
              "(see DESIGN.md for how it would shard); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_kv_cache_amd as lib
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(bits):
        return up(bits.view(np.int16)).view(torch.bfloat16)

    # ---- decode workload: config 3 (ctx 32768, 1 sequence, random pages)
    dec = workloads.config_case(3)
    dec_data = dec.all_data()
    k, v, q, slots = dec_data
    ctx = dec.max_context_len
    base = lib.alloc_cache(dec.num_pages, dec.n_kv_heads, dev)
    lib.kv_quant_write(up(k), up(v), up(slots), base)
    copies = [base] + [lib.PagedCache(base.k_cache.clone(), base.v_cache.clone(),
                                      base.k_scale.clone(), base.v_scale.clone(),
                                      base.num_pages, base.n_kv_heads)
                       for _ in range(args.decode_copies - 1)]
    q_dec = bf16(q[:, 0])                                   # [1, 24, 256]
    table = up(dec.block_table)
    ctx_t = up(dec.context_lens)
    k_new, v_new, slot_new = up(k[-1:]), up(v[-1:]), up(slots[-1:])
    out_dec = torch.empty((1, dec.n_q_heads, dec.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(lib.attn_decode_workspace_bytes(1, ctx, dec.n_q_heads), dtype=torch.uint8,
                     device=dev)

    # ---- prefill workload: config 4 (2048 new queries at ctx 32768, causal)
    pf = workloads.config_case(4)
    pf_data = pf.data()
    k4, v4, q4, slots4 = pf_data
    pos0 = pf.context_len - pf.n_new
    pcache = lib.alloc_cache(pf.num_pages, pf.n_kv_heads, dev)
    lib.kv_quant_write(up(k4[:pos0]), up(v4[:pos0]), up(slots4[:pos0]), pcache)
    k_chunk, v_chunk, s_chunk = up(k4[pos0:]), up(v4[pos0:]), up(slots4[pos0:])
    q_pf = bf16(q4)
    ptable = up(pf.block_table)
    out_pf = torch.empty((pf.n_new, pf.n_q_heads, pf.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    n_ev = 5
    R = len(copies)   # decode calls per step, one per cache copy (back to back)
    steps_total = args.warmup + args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps_total)]

    def step(i):
        ev = events[i]
        ev[0].record()
        lib.kv_quant_write(k_chunk, v_chunk, s_chunk, pcache)
        ev[1].record()
        lib.attn_prefill_chunk(q_pf, pcache, ptable, pf.context_len, True, out=out_pf)
        ev[2].record()
        for c in copies:
            lib.kv_quant_write(k_new, v_new, slot_new, c)
        ev[3].record()
        for c in copies:
            lib.attn_decode(q_dec, c, table, ctx_t, ctx, out=out_dec, workspace=ws)
        ev[4].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, steps_total):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def mean_ms(a, b):
        return float(np.mean([events[i][a].elapsed_time(events[i][b])
                              for i in range(args.warmup, steps_total)]))

    qw_chunk_ms, pf_ms = mean_ms(0, 1), mean_ms(1, 2)
    qw_tok_ms, dec_ms = mean_ms(2, 3) / R, mean_ms(3, 4) / R
    dec_b = decode_bytes(ctx, dec.n_q_heads, dec.n_kv_heads, dec.head_dim)
    pf_ops = prefill_ops(pf.context_len, pf.n_new, pf.n_q_heads, pf.head_dim)
    qw_b = quant_write_bytes(pf.n_new, pf.n_kv_heads, pf.head_dim)
    dec_gbps = dec_b / (dec_ms * 1e-3) / 1e9
    pf_tops = pf_ops / (pf_ms * 1e-3) / 1e12
    qw_gbps = qw_b / (qw_chunk_ms * 1e-3) / 1e9

    res = {
        "metric": "decode attn us/call + HBM GB/s at 32k ctx; prefill-chunk int8 TOPS (MFMA util)",
        "value": round(dec_ms * 1e3, 3),
        "unit": "us/call",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded N(0,1) K/V/Q, K outlier channels x10 in the chunk; random page tables)",
        "config": {"workload": "decode ctx=32768 (1 seq, 24q/4kv, d256, 64 partitions of 512, "
                               "MALL-cold over %d cache copies) + causal prefill chunk 2048 q at "
                               "ctx=32768 (30720 cached) + kv_quant_write of 2048+1 rows"
                               % len(copies),
                   "decode_ctx": ctx, "prefill_ctx": pf.context_len, "prefill_n_new": pf.n_new,
                   "n_q_heads": 24, "n_kv_heads": 4, "head_dim": 256, "page": 16,
                   "partition": 512},
        "decode_us": round(dec_ms * 1e3, 3),
        "decode_hbm_GBps": round(dec_gbps, 1),
        "prefill_ms": round(pf_ms, 4),
        "prefill_int8_TOPS": round(pf_tops, 1),
        "prefill_mfma_util": round(pf_tops / INT8_PEAK_TOPS, 4),
        "quant_write_2048_us": round(qw_chunk_ms * 1e3, 3),
        "quant_write_GBps": round(qw_gbps, 1),
        "quant_write_1tok_us": round(qw_tok_ms * 1e3, 3),
        "decode_calls_per_step": R,
        "roofline": {"bound": "mfma", "kernel": "prefill_chunk_kernel",
                     "achieved": round(pf_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
                     "frac": round(pf_tops / INT8_PEAK_TOPS, 4),
                     "per_launch": pf_ops, "traffic": recorded_traffic("prefill")},
        "roofline_decode": {"bound": "hbm", "kernel": "attn_decode (split + merge)",
                            "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "per_launch": dec_b,
                            "traffic": recorded_traffic("decode")},
    }
    # ---- the next rows on the same caches (not part of the step): multi-row verify
    # (nq query rows per sequence, fp32-class weights) and the int8-P decode, each timed
    # as groups of back-to-back calls over the MALL-cold copies.
    def group_us(fn, reps=10):
        for c in copies:
            fn(c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            for c in copies:
                fn(c)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(copies))

    rng = np.random.default_rng(11)
    verify = {}
    for nq in (2, 4, 8):
        qv = bf16(workloads.f32_to_bf16_bits(
            rng.standard_normal((1, nq, dec.n_q_heads, dec.head_dim), dtype=np.float32)))
        ov = torch.empty((1, nq, dec.n_q_heads, dec.head_dim), dtype=torch.float32, device=dev)
        wsv = torch.empty(lib.attn_verify_workspace_bytes(1, nq, ctx, dec.n_q_heads),
                          dtype=torch.uint8, device=dev)
        us = group_us(lambda c: lib.attn_verify(qv, c, table, ctx_t, ctx, out=ov, workspace=wsv))
        verify[f"nq{nq}"] = {"us": round(us, 3), "hbm_GBps": round(dec_b / (us * 1e-6) / 1e9, 1)}
    part = lib.attn_decode_partition_rows(1, ctx, dec.n_kv_heads)
    ws8 = torch.empty(lib.attn_decode_int8p_workspace_bytes(1, 1, ctx, dec.n_q_heads, dec.n_kv_heads),
                      dtype=torch.uint8, device=dev)
    i8p_us = group_us(lambda c: lib.attn_decode_int8p(q_dec, c, table, ctx_t, ctx, out=out_dec,
                                                      workspace=ws8))
    # short chunks at the end of the prefill context (the last n query rows): the split
    # route (key partitions + merge, or the int8-P decode kernel for n <= 8) against the
    # one pass; both stream the whole int8 K/V of the head group
    short = {}
    ws_sp = torch.empty(max(lib.attn_prefill_chunk_split_workspace_bytes(
        256, pf.context_len, True, pf.n_q_heads, pf.n_kv_heads), 256), dtype=torch.uint8,
        device=dev)
    for n in (1, 16, 64, 256):
        qn = q_pf[-n:]
        on = torch.empty((n, pf.n_q_heads, pf.head_dim), dtype=torch.float32, device=dev)
        t_split = group_us(lambda c: lib.attn_prefill_chunk_split(
            qn, pcache, ptable, pf.context_len, True, out=on, workspace=ws_sp))
        t_one = group_us(lambda c: lib.attn_prefill_chunk(qn, pcache, ptable, pf.context_len,
                                                          True, out=on), reps=2)
        ops = prefill_ops(pf.context_len, n, pf.n_q_heads, pf.head_dim)
        kv_b = decode_bytes(pf.context_len, pf.n_q_heads, pf.n_kv_heads, pf.head_dim)
        short[f"n{n}"] = {"split_us": round(t_split, 2), "one_pass_us": round(t_one, 1),
                          "int8_TOPS": round(ops / (t_split * 1e-6) / 1e12, 1),
                          "kv_GBps": round(kv_b / (t_split * 1e-6) / 1e9, 1)}
    # the fused producer (RoPE on Q/K, Q/K/V quantized, K/V paged write) for the chunk's
    # 2,048 tokens and for one decode token, bf16 inputs as a projection would give them
    qb = q_pf                                            # bf16 [2048, 24, 256]
    kb = bf16(workloads.f32_to_bf16_bits(k4[pos0:]))
    vb = bf16(workloads.f32_to_bf16_bits(v4[pos0:]))
    pos_t = torch.arange(pos0, pf.context_len, dtype=torch.int32, device=dev)
    rope_tab = up(workloads.rope_table(pf.context_len, pf.head_dim))
    prod_bytes = pf.n_new * (2 * pf.head_dim * (pf.n_q_heads + 2 * pf.n_kv_heads)
                             + pf.head_dim * (pf.n_q_heads + 2 * pf.n_kv_heads)
                             + 4 * (pf.n_q_heads + 2 * pf.n_kv_heads) + 8)
    for _ in range(3):
        lib.kv_produce(qb, kb, vb, pos_t, rope_tab, s_chunk, pcache)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        lib.kv_produce(qb, kb, vb, pos_t, rope_tab, s_chunk, pcache)
    e1.record()
    torch.cuda.synchronize()
    prod_us = e0.elapsed_time(e1) * 1e3 / 20
    # one decode token: the eager Python call costs more host time than the kernel takes,
    # so 8 calls are captured once in a graph and the graph is replayed
    one = (qb[-1:], kb[-1:], vb[-1:], pos_t[-1:], rope_tab, s_chunk[-1:], pcache)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.kv_produce(*one)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(8):
            lib.kv_produce(*one)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    tok1 = e0.elapsed_time(e1) * 1e3 / 160
    res["produce_2048"] = {"us": round(prod_us, 3), "bytes": prod_bytes,
                           "hbm_GBps": round(prod_bytes / (prod_us * 1e-6) / 1e9, 1),
                           "one_token_us_graph": round(tok1, 3)}
    # the high-precision route of a chunk with no history: bf16 attention of the chunk's
    # 2,048 rotated rows over themselves (causal)
    qr, kr = lib.kv_produce(qb, kb, vb, pos_t - pos0, rope_tab, s_chunk, pcache, rotated_bf16=True)
    out_fc = torch.empty_like(out_pf)
    ws_fc = torch.empty(max(lib.attn_chunk_bf16_workspace_bytes(pf.n_new, True, pf.n_q_heads,
                                                                pf.n_kv_heads), 256),
                        dtype=torch.uint8, device=dev)

    def fc_time(split):
        for _ in range(3):
            lib.attn_chunk_bf16(qr, kr, vb, True, out=out_fc, workspace=ws_fc, split=split)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            lib.attn_chunk_bf16(qr, kr, vb, True, out=out_fc, workspace=ws_fc, split=split)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 10
    fc_ms, fc_one_ms = fc_time(True), fc_time(False)
    n_fc = pf.n_new
    fc_flops = pf.n_q_heads * n_fc * (n_fc + 1) // 2 * 4 * pf.head_dim
    res["first_chunk_bf16_2048"] = {"ms": round(fc_ms, 4), "one_pass_ms": round(fc_one_ms, 4),
                                    "flops": fc_flops,
                                    "TFLOPs": round(fc_flops / (fc_ms * 1e-3) / 1e12, 1),
                                    "bf16_mfma_frac": round(fc_flops / (fc_ms * 1e-3) / 2.5e15, 4)}
    res["verify_ctx32768"] = verify
    res["decode_int8p_ctx32768"] = {"us": round(i8p_us, 3), "partition": part,
                                    "hbm_GBps": round(dec_b / (i8p_us * 1e-6) / 1e9, 1)}
    res["prefill_short_chunks_ctx32768"] = short
    # ---- spread of the per-step event times, MALL-warm and graph-replayed decode, and
    # ceilings measured on this machine (a 1 GiB device copy; hipBLASLt's int8 GEMM)
    dec_steps = [events[i][3].elapsed_time(events[i][4]) * 1e3 / R
                 for i in range(args.warmup, steps_total)]
    pf_steps = [events[i][1].elapsed_time(events[i][2]) for i in range(args.warmup, steps_total)]
    res["decode_us_spread"] = {"median": round(float(np.median(dec_steps)), 3),
                               "min": round(min(dec_steps), 3), "max": round(max(dec_steps), 3)}
    res["prefill_ms_spread"] = {"median": round(float(np.median(pf_steps)), 4),
                                "min": round(min(pf_steps), 4), "max": round(max(pf_steps), 4)}

    def per_call_us(fn, calls, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * calls)

    def warm8():
        for _ in range(R):
            lib.attn_decode(q_dec, base, table, ctx_t, ctx, out=out_dec, workspace=ws)
    warm_us = per_call_us(warm8, R)
    # kv_quant_write of a whole 32,768-token context in one call (fp32 rows in): the
    # HBM-bound regime of the writer, against the 2,048-row call of the step
    k_all, v_all, s_all = up(k4), up(v4), up(slots4)
    qw_big_us = per_call_us(lambda: lib.kv_quant_write(k_all, v_all, s_all, pcache), 1, reps=10)
    qw_big_b = quant_write_bytes(pf.context_len, pf.n_kv_heads, pf.head_dim)
    res["quant_write_32768"] = {"us": round(qw_big_us, 2), "bytes": qw_big_b,
                                "hbm_GBps": round(qw_big_b / (qw_big_us * 1e-6) / 1e9, 1)}
    del k_all, v_all, s_all
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in copies:
            lib.attn_decode(q_dec, c, table, ctx_t, ctx, out=out_dec, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        for c in copies:
            lib.attn_decode(q_dec, c, table, ctx_t, ctx, out=out_dec, workspace=ws)
    graph_us = per_call_us(dgraph.replay, R)
    # the other decode workloads: configs 1 and 2 (one sequence, ctx 256 and 3,328; eager
    # calls and 16 calls replayed from a graph) and config 5 (64 sequences, contexts
    # log-uniform in [1,024, 131,072], 3.6 GB of K/V: MALL-cold by size). Config 5's K/V
    # rows are drawn on the GPU (N(0,1)) into the config's page tables: the decode time
    # does not depend on the values.
    def decode_graph_us(call, n_calls=16):
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            call()
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_calls):
                call()
        return per_call_us(g.replay, n_calls)

    dcfg = {}
    for cfg in (1, 2):
        c = workloads.config_case(cfg)
        kk, vv, qq, ss = c.all_data()
        cc = lib.alloc_cache(c.num_pages, c.n_kv_heads, dev)
        lib.kv_quant_write(up(kk), up(vv), up(ss), cc)
        qd, tb, cl = bf16(qq[:, 0]), up(c.block_table), up(c.context_lens)
        od = torch.empty((c.num_seqs, c.n_q_heads, c.head_dim), dtype=torch.float32, device=dev)
        wd = torch.empty(max(lib.attn_decode_workspace_bytes(c.num_seqs, c.max_context_len,
                                                             c.n_q_heads), 256),
                         dtype=torch.uint8, device=dev)

        def call(qd=qd, cc=cc, tb=tb, cl=cl, c=c, od=od, wd=wd):
            lib.attn_decode(qd, cc, tb, cl, c.max_context_len, out=od, workspace=wd)
        eager = per_call_us(lambda: [call() for _ in range(16)], 16)
        graph = decode_graph_us(call)
        nbytes = decode_bytes(c.max_context_len, c.n_q_heads, c.n_kv_heads, c.head_dim)
        dcfg[f"config{cfg}"] = {"ctx": c.max_context_len, "bytes": nbytes,
                                "us_eager": round(eager, 3), "us_graph": round(graph, 3),
                                "GBps_graph": round(nbytes / (graph * 1e-6) / 1e9, 1)}
    c5 = workloads.config_case(5)
    cache5 = lib.alloc_cache(c5.num_pages, c5.n_kv_heads, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(c5.seed)
    for s_ in range(c5.num_seqs):
        sl5 = up(c5.seq_slots(s_))
        for t0 in range(0, int(c5.context_lens[s_]), 65536):
            nrow = min(65536, int(c5.context_lens[s_]) - t0)
            shp = (nrow, c5.n_kv_heads, c5.head_dim)
            lib.kv_quant_write(torch.randn(shp, generator=gen, device=dev),
                               torch.randn(shp, generator=gen, device=dev), sl5[t0:t0 + nrow],
                               cache5)
    q5 = torch.randn((c5.num_seqs, c5.n_q_heads, c5.head_dim), generator=gen,
                     device=dev).to(torch.bfloat16)
    tb5, cl5 = up(c5.block_table), up(c5.context_lens)
    o5 = torch.empty((c5.num_seqs, c5.n_q_heads, c5.head_dim), dtype=torch.float32, device=dev)
    w5 = torch.empty(lib.attn_decode_workspace_bytes(c5.num_seqs, c5.max_context_len,
                                                     c5.n_q_heads), dtype=torch.uint8, device=dev)
    t5 = per_call_us(lambda: lib.attn_decode(q5, cache5, tb5, cl5, c5.max_context_len, out=o5,
                                             workspace=w5), 1, reps=10)
    b5 = sum(decode_bytes(int(x), c5.n_q_heads, c5.n_kv_heads, c5.head_dim) for x in c5.context_lens)
    dcfg["config5"] = {"seqs": c5.num_seqs, "total_ctx": c5.total_tokens, "bytes": b5,
                       "us": round(t5, 2), "hbm_GBps": round(b5 / (t5 * 1e-6) / 1e9, 1),
                       "frac_of_8TBps": round(b5 / (t5 * 1e-6) / 8e12, 4)}
    del cache5, w5
    res["decode_configs"] = dcfg
    # one chunked-prefill step end to end (producer: RoPE, quantization and paged write of
    # the new rows; then the int8 chunk on the split route) for the last 64 and 256 rows
    # of the 32,768-token prefill context; it rewrites those rows' pages, so it runs last
    steps_e2e = {}
    for n in (64, 256):
        sl = slice(pf.n_new - n, pf.n_new)
        ws_st = torch.empty(lib.prefill_step_workspace_bytes(n, pf.context_len, pf.n_q_heads,
                                                             pf.n_kv_heads), dtype=torch.uint8,
                            device=dev)
        o_st = torch.empty((n, pf.n_q_heads, pf.head_dim), dtype=torch.float32, device=dev)
        args_st = (qb[sl], kb[sl], vb[sl], pos_t[sl], rope_tab, s_chunk[sl], pcache, ptable,
                   pf.context_len)
        t_st = per_call_us(lambda: lib.prefill_step(*args_st, out=o_st, workspace=ws_st), 1,
                           reps=10)
        # (eager calls at 64 rows are bound by the Python wrapper's argument checks; the
        # graph replay shows the GPU time)
        t_gr = decode_graph_us(lambda: lib.prefill_step(*args_st, out=o_st, workspace=ws_st),
                               n_calls=4)
        steps_e2e[f"n{n}"] = {"us_eager": round(t_st, 2), "us_graph": round(t_gr, 2)}
    res["prefill_step_ctx32768"] = steps_e2e
    res["decode_us_mall_warm"] = round(warm_us, 3)
    res["decode_us_graph"] = round(graph_us, 3)
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_GBps = 2 * nb / (per_call_us(lambda: dst.copy_(src), 1, reps=5) * 1e-6) / 1e9
    del src, dst
    try:
        ga = torch.randint(-127, 128, (8192, 8192), dtype=torch.int8, device=dev)
        gb = torch.randint(-127, 128, (8192, 8192), dtype=torch.int8, device=dev)
        gemm_TOPS = 2 * 8192 ** 3 / (per_call_us(lambda: torch._int_mm(ga, gb), 1, reps=5) * 1e-6) / 1e12
        del ga, gb
    except (RuntimeError, AttributeError):
        gemm_TOPS = None
    res["measured_ceilings"] = {
        "device_copy_GBps": round(copy_GBps, 1),
        "decode_frac_of_copy": round(dec_gbps / copy_GBps, 4),
        "int8_gemm_TOPS": None if gemm_TOPS is None else round(gemm_TOPS, 1),
        "prefill_frac_of_int8_gemm": None if gemm_TOPS is None else round(pf_tops / gemm_TOPS, 4)}
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        cb = cpu_baseline(dec, dec_data, pf, pf_data, args.cpu_budget)
        res["cpu_baseline"] = cb["decode"]
        res["cpu_baseline_prefill"] = cb["prefill"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
