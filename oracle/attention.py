"""Exact softmax attention over dequantized INT8 K/V (oracle). Test infrastructure only.

Definitions followed:
  * score = (Q_deq . K_deq) * sm_scale with sm_scale = 1/sqrt(d), and the output is
    softmax(score) @ V_deq ("INT8 KV and INT8 MMAC attention on a gfx936 DCU",
    §1.3: Score = QK^T * sQ * sK / sqrt(d); the int8 product times the two scales
    equals the product of the dequantized rows exactly);
  * GQA: query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * causal visibility: query token t sees keys 0 .. last_key[t] inclusive, where a
    chunk of n_new queries at the tail of a context of ctx keys has
    last_key[t] = ctx - n_new + t ("dot4-flash-attention" README, recthist prefix /
    causal tail: prefix keys fully visible, tail keys checked k <= q_offset + q);
  * decode split-K: keys cut into partitions of 512 rows, each reduced to a partial
    state (m, l, o), merged by log-sum-exp ("dot4-flash-attention" README route table:
    split-K stage 1 over 512-row splits, stage 2 merge; gfx936 article §3.3:
    per-partition work then a merge of softmax states and outputs);
  * int8 P (§3.3 of the gfx936 article): the softmax weight is multiplied by the
    key's V scale, then quantized per query row and per aligned 64-key block with
    scale = block absmax / 127; the block's int8 product with the V codes is scaled
    back by that block scale. The denominator is the sum of unquantized weights.

Everything is float64. The exact definition is the un-tiled one: one max over all
visible keys, one normalisation.
"""
from __future__ import annotations

import math

import numpy as np

from .quant import dequantize


def _check(qd, kd, vd):
    if qd.ndim != 3 or kd.ndim != 3 or vd.ndim != 3:
        raise ValueError("q [R,Hq,D], k/v [N,Hkv,D] expected")
    if qd.shape[1] % kd.shape[1]:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return qd.shape[1] // kd.shape[1]


def attention_exact(qd, kd, vd, sm_scale, last_key, *, row_chunk=128, return_stats=False):
    """Exact attention. qd [R,Hq,D], kd/vd [N,Hkv,D] float64; last_key [R] inclusive.

    Returns out [R,Hq,D] (and (m, l) [R,Hq] with m the max score, l = sum exp(s - m)).
    """
    qd = np.asarray(qd, np.float64); kd = np.asarray(kd, np.float64); vd = np.asarray(vd, np.float64)
    group = _check(qd, kd, vd)
    R, Hq, D = qd.shape
    N, Hkv, _ = kd.shape
    last_key = np.asarray(last_key, dtype=np.int64)
    out = np.empty((R, Hq, D), dtype=np.float64)
    m_all = np.empty((R, Hq)); l_all = np.empty((R, Hq))
    key_idx = np.arange(N)
    for g in range(Hkv):
        kg, vg = kd[:, g, :], vd[:, g, :]
        heads = slice(g * group, (g + 1) * group)
        for r0 in range(0, R, row_chunk):
            r1 = min(R, r0 + row_chunk)
            qg = qd[r0:r1, heads, :]                               # [r, group, D]
            r = r1 - r0
            s = (qg.reshape(r * group, D) @ kg.T).reshape(r, group, N) * sm_scale
            vis = key_idx[None, :] <= last_key[r0:r1, None]        # [r, N]
            s = np.where(vis[:, None, :], s, -np.inf)
            m = s.max(axis=-1)
            p = np.exp(s - m[..., None])
            l = p.sum(axis=-1)
            out[r0:r1, heads, :] = (p.reshape(r * group, N) @ vg).reshape(r, group, D) / l[..., None]
            m_all[r0:r1, heads] = m; l_all[r0:r1, heads] = l
    if return_stats:
        return out, m_all, l_all
    return out


def split_partials(qd_row, kd, vd, sm_scale, ctx, partition=512):
    """Decode stage-1 reference for one query token.

    qd_row [Hq,D]; keys 0..ctx-1. Partition j covers keys [j*partition,
    min((j+1)*partition, ctx)). Returns m [Hq,P], l [Hq,P], o [Hq,P,D] with
    o_j = sum_k exp(s_k - m_j) V_k (not normalised).
    """
    qd_row = np.asarray(qd_row, np.float64)
    group = qd_row.shape[0] // kd.shape[1]
    n_part = -(-ctx // partition)
    Hq, D = qd_row.shape
    m = np.empty((Hq, n_part)); l = np.empty((Hq, n_part)); o = np.empty((Hq, n_part, D))
    for h in range(Hq):
        g = h // group
        for j in range(n_part):
            a, b = j * partition, min((j + 1) * partition, ctx)
            s = kd[a:b, g, :] @ qd_row[h] * sm_scale
            m[h, j] = s.max()
            p = np.exp(s - m[h, j])
            l[h, j] = p.sum()
            o[h, j] = p @ vd[a:b, g, :]
    return m, l, o


def merge_partials(m, l, o):
    """Log-sum-exp merge of partial states: M = max m_j, L = sum l_j e^(m_j-M),
    out = sum o_j e^(m_j-M) / L. m, l [Hq,P]; o [Hq,P,D] -> [Hq,D]."""
    M = m.max(axis=-1, keepdims=True)
    w = np.exp(m - M)
    L = (l * w).sum(axis=-1)
    return (o * w[..., None]).sum(axis=1) / L[:, None]


def attention_int8p(qd, kd, v_codes, v_scales, sm_scale, last_key, *, block=64, row_chunk=64):
    """Int8-P emulation ("oracle B"): exact scores and softmax weights, then
    w = p * sV, per (row, aligned 64-key block) s_b = max w / 127, c = rint(w / s_b)
    (0 when s_b = 0), out = sum_b s_b * sum_k c_k * vcode_k / sum_k p_k.

    v_codes [N,Hkv,D] int8 and v_scales [N,Hkv] fp32 are the stored V.
    """
    qd = np.asarray(qd, np.float64); kd = np.asarray(kd, np.float64)
    vc = np.asarray(v_codes, np.float64)
    vs = np.asarray(v_scales, np.float64)
    group = _check(qd, kd, vc)
    R, Hq, D = qd.shape
    N, Hkv, _ = kd.shape
    last_key = np.asarray(last_key, dtype=np.int64)
    nb = -(-N // block)
    pad = nb * block - N
    key_idx = np.arange(N)
    out = np.empty((R, Hq, D))
    for g in range(Hkv):
        heads = slice(g * group, (g + 1) * group)
        vcg = np.concatenate([vc[:, g, :], np.zeros((pad, D))]).reshape(nb, block, D)
        vsg = vs[:, g]
        for r0 in range(0, R, row_chunk):
            r1 = min(R, r0 + row_chunk)
            r = r1 - r0
            s = (qd[r0:r1, heads, :].reshape(r * group, D) @ kd[:, g, :].T).reshape(r, group, N) * sm_scale
            vis = key_idx[None, :] <= last_key[r0:r1, None]
            s = np.where(vis[:, None, :], s, -np.inf)
            m = s.max(axis=-1, keepdims=True)
            p = np.exp(s - m)                                    # masked keys -> 0
            l = p.sum(axis=-1)
            w = p * vsg[None, None, :]
            w = np.concatenate([w, np.zeros(w.shape[:2] + (pad,))], axis=-1)
            w = w.reshape(w.shape[0], w.shape[1], nb, block)
            sb = w.max(axis=-1) / 127.0                          # [r, group, nb]
            safe = np.where(sb > 0, sb, 1.0)
            c = np.where(sb[..., None] > 0, np.rint(w / safe[..., None]), 0.0)
            acc = np.matmul(c.transpose(2, 0, 1, 3).reshape(nb, r * group, block), vcg)
            acc = acc.reshape(nb, r, group, D).transpose(1, 2, 0, 3)   # exact integer sums
            out[r0:r1, heads, :] = (acc * sb[..., None]).sum(axis=2) / l[..., None]
    return out


def decode_exact(q_codes, q_scales, cache_view, sm_scale):
    """Exact decode for one sequence from its gathered cache view.

    q_codes [Hq,D] int8, q_scales [Hq]; cache_view = (k_codes [ctx,Hkv,D], k_scales
    [ctx,Hkv], v_codes, v_scales). Returns [Hq,D] float64.
    """
    kc, ks, vc, vs = cache_view
    qd = dequantize(q_codes, q_scales)[None]
    ctx = kc.shape[0]
    return attention_exact(qd, dequantize(kc, ks), dequantize(vc, vs), sm_scale,
                           np.array([ctx - 1]))[0]


def verify_exact(q_codes, q_scales, cache_view, sm_scale):
    """Exact multi-row decode (speculative / multi-token verify) for one sequence.

    q_codes [nq,Hq,D] int8 and q_scales [nq,Hq] are the nq newest query rows; the
    cache view (k_codes [ctx,Hkv,D], k_scales [ctx,Hkv], v_codes, v_scales) already
    holds their K/V. Row i sits at position ctx - nq + i and sees keys 0 .. ctx - nq + i,
    the causal rule of a chunk ("dot4-flash-attention" README: the MTP verify step
    runs a few query rows at once and its next-steps list extends split-K decode to
    such small query batches; vLLM docs page, "Row shape routing": speculative-verify
    decode of a few rows runs on a multi-row kernel). A row with no visible key
    (ctx < nq) gets zeros. Returns [nq,Hq,D] float64.
    """
    kc, ks, vc, vs = cache_view
    nq = int(q_codes.shape[0])
    ctx = int(kc.shape[0])
    last = ctx - nq + np.arange(nq)
    out = np.zeros((nq,) + tuple(q_codes.shape[1:]), dtype=np.float64)
    live = last >= 0
    if live.any():
        qd = dequantize(q_codes[live], q_scales[live])
        out[live] = attention_exact(qd, dequantize(kc, ks), dequantize(vc, vs), sm_scale,
                                    last[live])
    return out


def verify_int8p(q_codes, q_scales, cache_view, sm_scale):
    """Int8-P decode / verify for one sequence ("oracle B" rule of attention_int8p with
    the verify visibility of verify_exact: row i of nq sees keys 0 .. ctx - nq + i; a row
    with no visible key gets zeros). The 64-key blocks are aligned to key 0, so the
    codes do not depend on how a kernel splits the keys ("INT8 KV and INT8 MMAC
    attention on a gfx936 DCU", §3.3: decode with INT8 PV, weights quantized per block
    with scale = block absmax / 127). Returns [nq,Hq,D] float64."""
    kc, ks, vc, vs = cache_view
    nq = int(q_codes.shape[0])
    ctx = int(kc.shape[0])
    last = ctx - nq + np.arange(nq)
    out = np.zeros((nq,) + tuple(q_codes.shape[1:]), dtype=np.float64)
    live = last >= 0
    if live.any():
        qd = dequantize(q_codes[live], q_scales[live])
        out[live] = attention_int8p(qd, dequantize(kc, ks), vc, vs, sm_scale, last[live])
    return out


def brute_force_attention(qd, kd, vd, sm_scale, last_key):
    """Pure-Python triple loop, for tiny shapes only (the pin of attention_exact)."""
    R, Hq, D = len(qd), len(qd[0]), len(qd[0][0])
    Hkv = len(kd[0])
    group = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(R)]
    for r in range(R):
        for h in range(Hq):
            g = h // group
            keys = range(int(last_key[r]) + 1)
            scores = []
            for k in keys:
                acc = 0.0
                for d in range(D):
                    acc += float(qd[r][h][d]) * float(kd[k][g][d])
                scores.append(acc * sm_scale)
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            for d in range(D):
                out[r][h][d] = sum(w * float(vd[k][g][d]) for w, k in zip(ws, keys)) / tot
    return np.array(out)


def brute_force_int8p(qd, kd, v_codes, v_scales, sm_scale, last_key, block=64):
    """Pure-Python loops of the int8-P emulation, tiny shapes only."""
    R, Hq, D = len(qd), len(qd[0]), len(qd[0][0])
    Hkv = len(kd[0])
    group = Hq // Hkv
    out = np.zeros((R, Hq, D))
    for r in range(R):
        for h in range(Hq):
            g = h // group
            n_vis = int(last_key[r]) + 1
            s = [sum(float(qd[r][h][d]) * float(kd[k][g][d]) for d in range(D)) * sm_scale
                 for k in range(n_vis)]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            l = sum(p)
            for b0 in range(0, n_vis, block):
                ks = range(b0, min(n_vis, b0 + block))
                w = [p[k] * float(v_scales[k][g]) for k in ks]
                sb = max(w) / 127.0
                for d in range(D):
                    tot = 0.0
                    for wk, k in zip(w, ks):
                        c = round(wk / sb) if sb > 0 else 0   # Python round: half to even
                        tot += c * int(v_codes[k][g][d])
                    out[r, h, d] += sb * tot
            out[r, h, :] /= l
    return out
