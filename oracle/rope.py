"""Rotary position embedding and the fused KV producer (oracle). Test infrastructure only.

The producer ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.2): after the Q/K/V
projections one kernel reads Q, K and V, applies RoPE to Q and K, reduces the absmax of
every row, computes the scales and codes, writes the K/V codes and scales into the paged
cache and keeps Q as int8 codes plus scale (no high-precision Q/K written back).

Readings where the article leaves a step open:
  * RoPE is the rotation of dimension pairs (i, i + rd/2), i < rd/2, of the first rd
    (rotary_dim) dimensions of a head by the angle of position pos and pair i; dims past
    rd pass through. The cos and sin of every (pos, i) come from a caller table
    cos_sin[pos] = [cos_0 .. cos_{rd/2-1}, sin_0 .. sin_{rd/2-1}] (fp32), so the
    frequencies, base and any scaling are the caller's;
  * the rotation is evaluated in fp32, every product and sum rounded on its own (no
    fused multiply-add): x_i' = fl(fl(x_i c_i) - fl(x_j s_i)),
    x_j' = fl(fl(x_j c_i) + fl(x_i s_i)), j = i + rd/2. The rotated rows are then
    quantized with the rule of `quant.quantize_rows`, so codes and scales are bit-exact
    functions of the inputs;
  * inputs are fp32, or bf16 widened exactly to fp32;
  * first chunk ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §3.1): a chunk with
    no history runs a high-precision attention while the producer still writes the int8
    K/V; that attention reads the rotated Q and K rounded to bf16 (nearest, ties to even)
    and the input V, the bf16 rows a high-precision kernel takes.
"""
from __future__ import annotations

import numpy as np

from . import paged, quant


def rope_rows(x, pos, cos_sin, rotary_dim):
    """Rotate rows. x [..., D] fp32, pos [...] int, cos_sin [max_pos, rotary_dim] fp32.

    Returns fp32 [..., D] by the pairwise fp32 rule above."""
    x = np.asarray(x, dtype=np.float32)
    rd = int(rotary_dim)
    half = rd // 2
    table = np.asarray(cos_sin, dtype=np.float32)[np.asarray(pos, dtype=np.int64)]  # [..., rd]
    c, s = table[..., :half], table[..., half:rd]
    a, b = x[..., :half], x[..., half:rd]
    out = x.copy()
    out[..., :half] = np.subtract(np.multiply(a, c, dtype=np.float32),
                                  np.multiply(b, s, dtype=np.float32), dtype=np.float32)
    out[..., half:rd] = np.add(np.multiply(b, c, dtype=np.float32),
                               np.multiply(a, s, dtype=np.float32), dtype=np.float32)
    return out


def produce(q, k, v, positions, cos_sin, rotary_dim, slots, cache):
    """The producer for one batch of T tokens: q [T,Hq,D], k/v [T,Hkv,D] fp32.

    Rotates q and k by each token's position, quantizes q, k and v per row, writes
    the k/v codes and scales at `slots` (paged.write_rows: a negative slot skips the
    token) and returns (q_codes int8 [T,Hq,D], q_scales fp32 [T,Hq])."""
    pos = np.asarray(positions, dtype=np.int64)
    qr = rope_rows(q, pos[:, None], cos_sin, rotary_dim)
    kr = rope_rows(k, pos[:, None], cos_sin, rotary_dim)
    qc, qs = quant.quantize_rows(qr)
    kc, ks = quant.quantize_rows(kr)
    vc, vs = quant.quantize_rows(v)
    paged.write_rows(cache, slots, kc, ks, vc, vs)
    return qc, qs


def produce_first_chunk(q, k, v, positions, cos_sin, rotary_dim, slots, cache):
    """The producer of a chunk with no history: the paged int8 K/V write of `produce`,
    and the rotated Q and K rows rounded to bf16 for the high-precision attention.
    Returns (q_rot bf16 bits [T,Hq,D], k_rot bf16 bits [T,Hkv,D])."""
    pos = np.asarray(positions, dtype=np.int64)
    qr = rope_rows(q, pos[:, None], cos_sin, rotary_dim)
    kr = rope_rows(k, pos[:, None], cos_sin, rotary_dim)
    kc, ks = quant.quantize_rows(kr)
    vc, vs = quant.quantize_rows(v)
    paged.write_rows(cache, slots, kc, ks, vc, vs)
    return quant.f32_to_bf16_rne(qr), quant.f32_to_bf16_rne(kr)
