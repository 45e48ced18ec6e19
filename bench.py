"""Benchmark of the INT8-KV attention hot path on one MI355X.

One step = every row of the path over one batch of synthetic input:
  1. kv_quant_write of the 2048 new rows of a causal prefill chunk (fp32 K/V in);
  2. attn_prefill_chunk: 2048 queries at the tail of a 32768-key context
     (30720 cached + 2048 new), 24 q / 4 KV heads, head_dim 256, int8 P per 64-key block;
  3. kv_quant_write of one new decode token into each of `--decode-copies` caches;
  4. attn_decode at context 32768 (split-K over 64 partitions of 512 rows + merge),
     once per cache copy, back to back. The copies are identical and are read in
     rotation, so no call finds its 68 MB working set in the 256 MB Infinity Cache
     (MALL-cold).

Timing:
  * the K timed steps run eagerly, bracketed by synchronisations (ms_per_step), with HIP
    events around each group of calls on the stream the library launches on; the
    prefill's event time is the `achieved` figure of the roofline (the dominant kernel);
  * the headline `value` (decode microseconds per call at ctx 32768) and the prefill and
    ceiling figures are also taken by the graph protocol: each workload is captured once
    in a HIP graph (decode: 32 calls, 4 rounds over the 8 MALL-cold copies), and 4
    repetitions are run interleaved across the workloads; each repetition replays the
    graph once untimed and then once timed with events, and the highest and lowest of the
    4 timed replays are dropped (the mean of the middle two is reported, with all four).
  * measured ceilings, in the same run and by the same protocol: the library's streaming
    read over 8 rotating buffers of the decode's size (and one large buffer), and its
    int8 MFMA loop; fractions are given of the spec peaks and of these.

Printed: one JSON line.
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
MFMA_I8_OPS = 16 * 16 * 64 * 2   # one v_mfma_i32_16x16x64_i8


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
    src = {"prefill": ["prefill.hip", "common.hpp"],
           "decode": ["decode.hip", "decode_item.inc", "common.hpp"]}[kind]
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


def trimmed(values):
    """4 repetitions: drop the highest and the lowest, mean of the middle two."""
    v = sorted(values)
    mid = v[1:-1] if len(v) > 2 else v
    return float(np.mean(mid)), [round(x, 4) for x in values]


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return model, len(os.sched_getaffinity(0)), blas


def cpu_baselines(budget_s: float):
    """The oracle as it stands, on the host's cores, for every workload (quantization timed
    apart from attention; attention from the codes):
      configs 1-3: whole decode calls; config 4: a sample of the chunk's query rows (exact
      attention and, on a smaller sample, the int8-P rule); config 5: a sample of its
      sequences, streamed (generate, quantize, attend), scaled to the whole batch by keys."""
    from oracle import attention, quant
    model, host_cores, blas = cpu_info()
    per = budget_s / 6.0
    out = {"cpu_model": model, "host_cores": host_cores, "blas_threads": blas}

    def timed(fn, max_calls=20, min_calls=1):
        calls, t0 = 0, time.perf_counter()
        while calls < min_calls or (time.perf_counter() - t0 < per and calls < max_calls):
            fn()
            calls += 1
        return (time.perf_counter() - t0) / calls, calls

    for cfg in (1, 2, 3):
        c = workloads.config_case(cfg)
        k, v, q, _ = c.all_data()
        t_q = time.perf_counter()
        kc, ks = quant.quantize_rows(k)
        vc, vs = quant.quantize_rows(v)
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q[0, 0]))
        t_q = time.perf_counter() - t_q
        view = (kc, ks, vc, vs)
        t_a, calls = timed(lambda: attention.decode_exact(qc, qs, view, workloads.SM_SCALE))
        out[f"config{cfg}"] = {"attention_us_per_call": round(t_a * 1e6, 1),
                               "quantize_us": round(t_q * 1e6, 1),
                               "sample": f"{calls} whole decode calls at ctx {c.max_context_len}; "
                                         f"quantization of its {c.max_context_len} K/V rows + Q"}
    # config 4: sampled query rows of the chunk, ops of the visible pairs they cover
    c4 = workloads.config_case(4)
    k4, v4, q4, _ = c4.data()
    t_q = time.perf_counter()
    kc4, ks4 = quant.quantize_rows(k4)
    vc4, vs4 = quant.quantize_rows(v4)
    qc4, qs4 = quant.quantize_rows(quant.bf16_bits_to_f32(q4))
    t_q = time.perf_counter() - t_q
    kd, vd = quant.dequantize(kc4, ks4), quant.dequantize(vc4, vs4)
    pos0 = c4.context_len - c4.n_new
    rng = np.random.default_rng(0)
    res4 = {}
    for name, fn, step in (("exact", lambda qd, rows: attention.attention_exact(
                                qd, kd, vd, workloads.SM_SCALE, pos0 + rows), 32),
                           ("int8p_rule", lambda qd, rows: attention.attention_int8p(
                                qd, kd, vc4, vs4, workloads.SM_SCALE, pos0 + rows), 8)):
        done, ops, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < per and done < c4.n_new:
            rows = np.sort(rng.choice(c4.n_new, step, replace=False))
            fn(quant.dequantize(qc4[rows], qs4[rows]), rows)
            done += step
            ops += int(np.sum(pos0 + rows + 1)) * c4.n_q_heads * 4 * c4.head_dim
        dt = time.perf_counter() - t0
        res4[name] = {"TOPS": round(ops / dt / 1e12, 6), "rows": done,
                      "ms_whole_chunk_est": round(prefill_ops(c4.context_len, c4.n_new,
                                                              c4.n_q_heads, c4.head_dim)
                                                  / (ops / dt) * 1e3, 1)}
    out["config4"] = {**res4, "quantize_us": round(t_q * 1e6, 1),
                      "sample": "random query rows of the 2048-row chunk (all 24 heads); "
                                "ms_whole_chunk_est scales by visible (row, key) pairs; "
                                "quantization of all 32768 K/V rows and 2048 Q rows"}
    # config 5: a sample of sequences at quantiles of the context length
    c5 = workloads.config_case(5)
    order = np.argsort(c5.context_lens)
    pick = [int(order[i]) for i in (0, len(order) // 3, 2 * len(order) // 3)]
    keys, t_qs, t_as = 0, 0.0, 0.0
    for s in pick:
        k, v, q = c5.seq_data(s)
        t0 = time.perf_counter()
        kc, ks = quant.quantize_rows(k)
        vc, vs = quant.quantize_rows(v)
        qc, qs = quant.quantize_rows(quant.bf16_bits_to_f32(q[0]))
        t1 = time.perf_counter()
        attention.decode_exact(qc, qs, (kc, ks, vc, vs), workloads.SM_SCALE)
        t2 = time.perf_counter()
        keys += int(c5.context_lens[s])
        t_qs += t1 - t0
        t_as += t2 - t1
        if t_qs + t_as > 2 * per:
            break
    scale = c5.total_tokens / keys
    out["config5"] = {"attention_us_per_call_est": round(t_as * scale * 1e6, 1),
                      "quantize_us_est": round(t_qs * scale * 1e6, 1),
                      "sample": f"sequences {pick[:len(pick)]} (contexts "
                                f"{[int(c5.context_lens[s]) for s in pick]}), streamed; "
                                f"scaled by keys to all {c5.num_seqs} sequences "
                                f"({c5.total_tokens} keys)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the rows after the step (verify, int8-P decode, short chunks, "
                         "producer, first chunk, other decode configs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, one device-to-device copy of this many MiB "
                         "(reference dispatch for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: it measures one GPU's share of the work "
              "(the library has no multi-GPU path); use --gpus 1", file=sys.stderr)
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
    k, v, q, slots = dec.all_data()
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
    del k, v, q

    # ---- prefill workload: config 4 (2048 new queries at ctx 32768, causal)
    pf = workloads.config_case(4)
    k4, v4, q4, slots4 = pf.data()
    pos0 = pf.context_len - pf.n_new
    pcache = lib.alloc_cache(pf.num_pages, pf.n_kv_heads, dev)
    lib.kv_quant_write(up(k4[:pos0]), up(v4[:pos0]), up(slots4[:pos0]), pcache)
    k_chunk, v_chunk, s_chunk = up(k4[pos0:]), up(v4[pos0:]), up(slots4[pos0:])
    q_pf = bf16(q4)
    ptable = up(pf.block_table)
    out_pf = torch.empty((pf.n_new, pf.n_q_heads, pf.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    dec_b = decode_bytes(ctx, dec.n_q_heads, dec.n_kv_heads, dec.head_dim)
    pf_ops = prefill_ops(pf.context_len, pf.n_new, pf.n_q_heads, pf.head_dim)

    # ---- the timed steps (eager; events around each group of calls)
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
    qw_tok_ms, dec_eager_ms = mean_ms(2, 3) / R, mean_ms(3, 4) / R
    dec_steps = [events[i][3].elapsed_time(events[i][4]) * 1e3 / R
                 for i in range(args.warmup, steps_total)]
    pf_steps = [events[i][1].elapsed_time(events[i][2]) for i in range(args.warmup, steps_total)]

    # ---- the graph protocol: decode, prefill and the measured ceilings
    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    rounds = 4
    read_bufs = [torch.empty(-(-dec_b // 16) * 16, dtype=torch.uint8, device=dev).fill_(i + 1)
                 for i in range(R)]
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    sink = torch.zeros(4 * 8192, dtype=torch.int32, device=dev)

    def per_call_eager(fn, calls):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    # the streaming read's workgroup count is the best of a short sweep (a ceiling)
    read_wg = min((512, 1024, 2048, 4096), key=lambda n: per_call_eager(
        lambda: [lib.ceiling_stream_read(b, n, sink) for b in read_bufs * 2], 2 * R))
    # the page-gather read (the decode's own access pattern): pages per workgroup likewise
    n_blk = -(-ctx // 16)
    gather_ppw = min((8, 16, 32), key=lambda n: per_call_eager(
        lambda: [lib.ceiling_page_gather(c, table, n_blk, n, sink) for c in copies * 2], 2 * R))
    gather_b = n_blk * (dec.n_kv_heads * (2 * 4096 + 2 * 64) + 4)
    mfma_wg, mfma_iters = 1024, 2000
    mfma_count = lib.lib().int8attn_ceiling_mfma_i8_count(mfma_wg, mfma_iters)

    work = {
        "decode": (lambda: [lib.attn_decode(q_dec, c, table, ctx_t, ctx, out=out_dec, workspace=ws)
                            for _ in range(rounds) for c in copies], rounds * R),
        "prefill": (lambda: lib.attn_prefill_chunk(q_pf, pcache, ptable, pf.context_len, True,
                                                   out=out_pf), 1),
        "read_decode_size": (lambda: [lib.ceiling_stream_read(b, read_wg, sink)
                                      for _ in range(rounds) for b in read_bufs], rounds * R),
        "read_1GiB": (lambda: lib.ceiling_stream_read(big, 4096, sink), 1),
        "page_gather": (lambda: [lib.ceiling_page_gather(c, table, n_blk, gather_ppw, sink)
                                 for _ in range(rounds) for c in copies], rounds * R),
        "mfma_i8": (lambda: lib.ceiling_mfma_i8(mfma_wg, mfma_iters, sink), 1),
    }
    graphs = {name: (capture(fn), n) for name, (fn, n) in work.items()}
    reps = {name: [] for name in graphs}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(4):
        for name, (g, n) in graphs.items():
            g.replay()                  # untimed, straight into the timed replay
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            reps[name].append(e0.elapsed_time(e1) * 1e3 / n)   # us per call
    dec_us, dec_reps = trimmed(reps["decode"])
    pf_graph_ms, pf_reps = trimmed([x / 1e3 for x in reps["prefill"]])
    rd_us, rd_reps = trimmed(reps["read_decode_size"])
    big_us, _ = trimmed(reps["read_1GiB"])
    mf_us, mf_reps = trimmed(reps["mfma_i8"])
    ga_us, ga_reps = trimmed(reps["page_gather"])
    read_ceiling = dec_b / (rd_us * 1e-6) / 1e9          # GB/s for the decode's bytes
    read_1g = (1 << 30) / (big_us * 1e-6) / 1e9
    mfma_ceiling = mfma_count * MFMA_I8_OPS / (mf_us * 1e-6) / 1e12
    del read_bufs, big

    dec_gbps = dec_b / (dec_us * 1e-6) / 1e9
    pf_tops = pf_ops / (pf_ms * 1e-3) / 1e12
    pf_tops_graph = pf_ops / (pf_graph_ms * 1e-3) / 1e12
    qw_b = quant_write_bytes(pf.n_new, pf.n_kv_heads, pf.head_dim)

    res = {
        "metric": "decode attn us/call + HBM GB/s at 32k ctx; prefill-chunk int8 TOPS (MFMA util)",
        "value": round(dec_us, 3),
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
        "timing": "value: decode per call from a HIP graph of 32 MALL-cold calls, 4 "
                  "interleaved repetitions, high and low dropped; roofline.achieved: the "
                  "prefill's event time in the eager timed steps",
        "decode_us": round(dec_us, 3),
        "decode_us_reps": dec_reps,
        "decode_hbm_GBps": round(dec_gbps, 1),
        "decode_us_eager": round(dec_eager_ms * 1e3, 3),
        "decode_us_eager_spread": {"median": round(float(np.median(dec_steps)), 3),
                                   "min": round(min(dec_steps), 3), "max": round(max(dec_steps), 3)},
        "prefill_ms": round(pf_ms, 4),
        "prefill_ms_spread": {"median": round(float(np.median(pf_steps)), 4),
                              "min": round(min(pf_steps), 4), "max": round(max(pf_steps), 4)},
        "prefill_ms_graph": round(pf_graph_ms, 4),
        "prefill_ms_graph_reps": pf_reps,
        "prefill_int8_TOPS": round(pf_tops, 1),
        "prefill_mfma_util": round(pf_tops / INT8_PEAK_TOPS, 4),
        "quant_write_2048_us": round(qw_chunk_ms * 1e3, 3),
        "quant_write_GBps": round(qw_b / (qw_chunk_ms * 1e-3) / 1e9, 1),
        "quant_write_1tok_us": round(qw_tok_ms * 1e3, 3),
        "decode_calls_per_step": R,
        "measured_ceilings": {
            "stream_read_decode_size_GBps": round(read_ceiling, 1),
            "stream_read_decode_size_us": round(rd_us, 3),
            "stream_read_decode_size_reps_us": rd_reps,
            "stream_read_workgroups": read_wg,
            "stream_read_1GiB_GBps": round(read_1g, 1),
            "page_gather_decode_us": round(ga_us, 3),
            "page_gather_decode_GBps": round(gather_b / (ga_us * 1e-6) / 1e9, 1),
            "page_gather_decode_reps_us": ga_reps,
            "page_gather_pages_per_workgroup": gather_ppw,
            "mfma_i8_TOPS": round(mfma_ceiling, 1),
            "mfma_i8_reps_us": mf_reps,
            "mfma_i8_count": int(mfma_count),
            "note": "library kernels int8attn_ceiling_stream_read (16-byte loads, the decode's "
                    "68 MB over 8 rotating buffers, MALL-cold), int8attn_ceiling_page_gather "
                    "(the decode's K/V pages and scales through its block table, over the same "
                    "cache copies) and int8attn_ceiling_mfma_i8 (8 independent "
                    "v_mfma_i32_16x16x64_i8 chains per wave), same protocol"},
        "roofline": {"bound": "mfma", "kernel": "prefill_chunk_kernel",
                     "achieved": round(pf_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
                     "frac": round(pf_tops / INT8_PEAK_TOPS, 4),
                     "frac_of_measured": round(pf_tops / mfma_ceiling, 4),
                     "measured_peak": round(mfma_ceiling, 1),
                     "per_launch": pf_ops, "traffic": recorded_traffic("prefill")},
        "roofline_decode": {"bound": "hbm", "kernel": "attn_decode (split + merge)",
                            "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                            "frac_of_measured": round(dec_gbps / read_ceiling, 4),
                            "measured_peak": round(read_ceiling, 1),
                            "frac_of_page_gather": round(ga_us / dec_us, 4),
                            "per_launch": dec_b, "traffic": recorded_traffic("decode")},
    }

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

    def graph_us(call, n_calls=16):
        g = capture(lambda: [call() for _ in range(n_calls)])
        return per_call_us(g.replay, n_calls)

    # the chunk's writer without the launch gaps of an eager call (8 calls per graph)
    qw_graph_us = graph_us(lambda: lib.kv_quant_write(k_chunk, v_chunk, s_chunk, pcache), n_calls=8)
    res["quant_write_2048_us_graph"] = round(qw_graph_us, 3)
    res["quant_write_GBps_graph"] = round(qw_b / (qw_graph_us * 1e-6) / 1e9, 1)

    res["decode_us_mall_warm"] = round(per_call_us(
        lambda: [lib.attn_decode(q_dec, base, table, ctx_t, ctx, out=out_dec, workspace=ws)
                 for _ in range(R)], R), 3)
    if not args.no_next_rows:
        next_rows(res, lib, torch, dev, up, bf16, dec, pf, copies, table, ctx_t, ctx, q_dec,
                  out_dec, ws, dec_b, q_pf, pcache, ptable, out_pf, k4, v4, slots4, s_chunk,
                  pos0, per_call_us, graph_us)
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_GBps = 2 * nb / (per_call_us(lambda: dst.copy_(src), 1, reps=5) * 1e-6) / 1e9
    del src, dst
    res["library_references"] = {
        "device_copy_1GiB_GBps": round(copy_GBps, 1),
        "note": "torch's device-to-device copy (read + written bytes); context only, the "
                "ceilings are measured_ceilings"}
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        cb = cpu_baselines(args.cpu_budget)
        c3 = cb["config3"]
        res["cpu_baseline"] = {"value": c3["attention_us_per_call"], "unit": "us/call",
                               "cores": cb["blas_threads"] or cb["host_cores"], "kind": "oracle",
                               "sample": c3["sample"] + " (decode at ctx 32768, from the codes)",
                               "cpu_model": cb["cpu_model"], "host_cores": cb["host_cores"]}
        res["cpu_baseline_configs"] = cb
        gpu = {"config1": res.get("decode_configs", {}).get("config1", {}).get("us_graph"),
               "config2": res.get("decode_configs", {}).get("config2", {}).get("us_graph"),
               "config3": dec_us,
               "config4_ms": pf_ms,
               "config5": res.get("decode_configs", {}).get("config5", {}).get("us")}
        res["cpu_vs_gpu"] = {
            "config1_x": None if not gpu["config1"] else round(cb["config1"]["attention_us_per_call"] / gpu["config1"], 1),
            "config2_x": None if not gpu["config2"] else round(cb["config2"]["attention_us_per_call"] / gpu["config2"], 1),
            "config3_x": round(c3["attention_us_per_call"] / dec_us, 1),
            "config4_x": round(cb["config4"]["exact"]["ms_whole_chunk_est"] / pf_ms, 1),
            "config5_x": None if not gpu["config5"] else round(cb["config5"]["attention_us_per_call_est"] / gpu["config5"], 1)}
    print(json.dumps(res), flush=True)


def gpu_shares(lib, torch, dev, up, dec, copies, table, ctx, q_dec, graph_us):
    """Config 3's decode at one GPU's share of a sharded run, at the share's real shape:
    tensor parallel over 4 GPUs (one KV head and its 6 query heads, all 32,768 keys) and
    context parallel over 8 GPUs (4,096 of the keys, 8 partitions, all heads; the exchange
    and the cross-GPU merge are not part of it). MALL-cold: every call in a replay reads
    its own K/V (24 one-head caches of 17 MB; 64 disjoint 4,096-key windows of the 8 cache
    copies), graph-timed. The one-head K/V are drawn on the GPU (torch's generator), N(0,1)
    as in config 3."""
    import itertools
    D, page = dec.head_dim, workloads.PAGE
    t = np.arange(ctx)
    slots = up((dec.block_table[0, t // page].astype(np.int64) * page + t % page).astype(np.int32))
    gen = torch.Generator(device=dev)
    gen.manual_seed(dec.seed + 100)
    tp = []
    for _ in range(24):
        c1 = lib.alloc_cache(dec.num_pages, 1, dev)
        lib.kv_quant_write(torch.randn((ctx, 1, D), generator=gen, device=dev),
                           torch.randn((ctx, 1, D), generator=gen, device=dev), slots, c1)
        tp.append(c1)
    q_tp = q_dec[:, :6].contiguous()
    ctx1 = torch.full((1,), ctx, dtype=torch.int32, device=dev)
    o_tp = torch.empty((1, 6, D), dtype=torch.float32, device=dev)
    w_tp = torch.empty(lib.attn_decode_workspace_bytes(1, ctx, 6), dtype=torch.uint8, device=dev)
    it = itertools.cycle(tp)
    us_tp = graph_us(lambda: lib.attn_decode(q_tp, next(it), table, ctx1, ctx, out=o_tp,
                                             workspace=w_tp), n_calls=len(tp))
    b_tp = decode_bytes(ctx, 6, 1, D)
    n_cp = 4096
    wins = [(c, up(np.ascontiguousarray(dec.block_table[:, w * (n_cp // page):(w + 1) * (n_cp // page)])))
            for c in copies for w in range(ctx // n_cp)]
    ctx_cp = torch.full((1,), n_cp, dtype=torch.int32, device=dev)
    o_cp = torch.empty((1, dec.n_q_heads, D), dtype=torch.float32, device=dev)
    w_cp = torch.empty(lib.attn_decode_workspace_bytes(1, n_cp, dec.n_q_heads), dtype=torch.uint8,
                       device=dev)
    it2 = itertools.cycle(wins)

    def cp_call():
        c, tb = next(it2)
        lib.attn_decode(q_dec, c, tb, ctx_cp, n_cp, out=o_cp, workspace=w_cp)
    us_cp = graph_us(cp_call, n_calls=len(wins))
    b_cp = decode_bytes(n_cp, dec.n_q_heads, dec.n_kv_heads, D)
    del tp
    return {"tp4_1kv_6q_ctx32768": {"us": round(us_tp, 3), "bytes": b_tp,
                                    "hbm_GBps": round(b_tp / (us_tp * 1e-6) / 1e9, 1),
                                    "workgroups": ctx // 512},
            "cp8_4096_keys_4kv_24q": {"us": round(us_cp, 3), "bytes": b_cp,
                                      "hbm_GBps": round(b_cp / (us_cp * 1e-6) / 1e9, 1),
                                      "workgroups": (n_cp // 512) * dec.n_kv_heads},
            "note": "graph-timed, MALL-cold; one GPU's share of config 3's decode"}


def next_rows(res, lib, torch, dev, up, bf16, dec, pf, copies, table, ctx_t, ctx, q_dec, out_dec,
              ws, dec_b, q_pf, pcache, ptable, out_pf, k4, v4, slots4, s_chunk, pos0, per_call_us,
              graph_us):
    """The rows after the step on the same caches (not part of the step): multi-row verify
    and the int8-P decode over the MALL-cold copies, short chunks, the fused producer, the
    first-chunk bf16 route, the other decode configs and prefill_step end to end."""
    def group_us(fn, reps=10):
        return per_call_us(lambda: [fn(c) for c in copies], len(copies), reps)

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
    res["verify_ctx32768"] = verify
    part = lib.attn_decode_partition_rows(1, ctx, dec.n_kv_heads)
    ws8 = torch.empty(lib.attn_decode_int8p_workspace_bytes(1, 1, ctx, dec.n_q_heads, dec.n_kv_heads),
                      dtype=torch.uint8, device=dev)
    i8p_us = group_us(lambda c: lib.attn_decode_int8p(q_dec, c, table, ctx_t, ctx, out=out_dec,
                                                      workspace=ws8))
    res["decode_int8p_ctx32768"] = {"us": round(i8p_us, 3), "partition": part,
                                    "hbm_GBps": round(dec_b / (i8p_us * 1e-6) / 1e9, 1)}
    res["decode_one_gpu_shares"] = gpu_shares(lib, torch, dev, up, dec, copies, table, ctx,
                                              q_dec, graph_us)
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
    res["prefill_short_chunks_ctx32768"] = short
    # the fused producer (RoPE on Q/K, Q/K/V quantized, K/V paged write) for the chunk's
    # 2,048 tokens and for one decode token, bf16 inputs as a projection would give them
    qb = q_pf
    kb = bf16(workloads.f32_to_bf16_bits(k4[pos0:]))
    vb = bf16(workloads.f32_to_bf16_bits(v4[pos0:]))
    pos_t = torch.arange(pos0, pf.context_len, dtype=torch.int32, device=dev)
    rope_tab = up(workloads.rope_table(pf.context_len, pf.head_dim))
    prod_bytes = pf.n_new * (2 * pf.head_dim * (pf.n_q_heads + 2 * pf.n_kv_heads)
                             + pf.head_dim * (pf.n_q_heads + 2 * pf.n_kv_heads)
                             + 4 * (pf.n_q_heads + 2 * pf.n_kv_heads) + 8)
    prod_us = per_call_us(lambda: lib.kv_produce(qb, kb, vb, pos_t, rope_tab, s_chunk, pcache), 1,
                          reps=20)
    one = (qb[-1:], kb[-1:], vb[-1:], pos_t[-1:], rope_tab, s_chunk[-1:], pcache)
    tok1 = graph_us(lambda: lib.kv_produce(*one), n_calls=8)
    prod_graph_us = graph_us(lambda: lib.kv_produce(qb, kb, vb, pos_t, rope_tab, s_chunk, pcache),
                             n_calls=8)
    res["produce_2048"] = {"us": round(prod_us, 3), "bytes": prod_bytes,
                           "hbm_GBps": round(prod_bytes / (prod_us * 1e-6) / 1e9, 1),
                           "us_graph": round(prod_graph_us, 3),
                           "hbm_GBps_graph": round(prod_bytes / (prod_graph_us * 1e-6) / 1e9, 1),
                           "one_token_us_graph": round(tok1, 3)}
    # the high-precision route of a chunk with no history: bf16 attention of the chunk's
    # 2,048 rotated rows over themselves (causal)
    qr, kr = lib.kv_produce(qb, kb, vb, pos_t - pos0, rope_tab, s_chunk, pcache, rotated_bf16=True)
    out_fc = torch.empty_like(out_pf)
    ws_fc = torch.empty(max(lib.attn_chunk_bf16_workspace_bytes(pf.n_new, True, pf.n_q_heads,
                                                                pf.n_kv_heads), 256),
                        dtype=torch.uint8, device=dev)
    fc_ms = per_call_us(lambda: lib.attn_chunk_bf16(qr, kr, vb, True, out=out_fc, workspace=ws_fc),
                        1) / 1e3
    fc_one_ms = per_call_us(lambda: lib.attn_chunk_bf16(qr, kr, vb, True, out=out_fc, split=False),
                            1) / 1e3
    n_fc = pf.n_new
    fc_flops = pf.n_q_heads * n_fc * (n_fc + 1) // 2 * 4 * pf.head_dim
    res["first_chunk_bf16_2048"] = {"ms": round(fc_ms, 4), "one_pass_ms": round(fc_one_ms, 4),
                                    "flops": fc_flops,
                                    "TFLOPs": round(fc_flops / (fc_ms * 1e-3) / 1e12, 1),
                                    "bf16_mfma_frac": round(fc_flops / (fc_ms * 1e-3) / 2.5e15, 4)}
    # kv_quant_write of a whole 32,768-token context in one call (fp32 rows in)
    k_all, v_all, s_all = up(k4), up(v4), up(slots4)
    qw_big_us = per_call_us(lambda: lib.kv_quant_write(k_all, v_all, s_all, pcache), 1, reps=10)
    qw_big_b = quant_write_bytes(pf.context_len, pf.n_kv_heads, pf.head_dim)
    res["quant_write_32768"] = {"us": round(qw_big_us, 2), "bytes": qw_big_b,
                                "hbm_GBps": round(qw_big_b / (qw_big_us * 1e-6) / 1e9, 1)}
    del k_all, v_all, s_all
    # the other decode workloads: configs 1 and 2 (one sequence, ctx 256 and 3,328; eager
    # calls and 16 calls replayed from a graph) and config 5 (64 sequences, contexts
    # log-uniform in [1,024, 131,072], 3.6 GB of K/V: MALL-cold by size). Config 5's K/V
    # rows are drawn on the GPU (N(0,1)) into the config's page tables: the decode time
    # does not depend on the values (its parity test uses the seeded host rows).
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
        graph = graph_us(call)
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
        t_gr = graph_us(lambda: lib.prefill_step(*args_st, out=o_st, workspace=ws_st), n_calls=4)
        steps_e2e[f"n{n}"] = {"us_eager": round(t_st, 2), "us_graph": round(t_gr, 2)}
    res["prefill_step_ctx32768"] = steps_e2e


if __name__ == "__main__":
    main()
