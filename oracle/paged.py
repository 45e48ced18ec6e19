"""Paged INT8 KV cache: byte layout by index formula (oracle). Test infrastructure only.

The cache is a pool of pages of 16 tokens; a sequence's block table lists its pages
in token order; slot = page * 16 + offset ("INT8 KV and INT8 MMAC attention on a
gfx936 DCU", §2.3: paged K/V codes with FP32 scale arrays stored apart from the
codes; K and V may use different layouts, each arranged for 16-byte moves).

Byte offset of element (page p, kv head h, token offset o in 0..15, dim d in 0..255),
with H kv heads; every (p, h) owns one contiguous 4096-byte block in each array:

  K codes:  ((p*H + h) * 16 + d // 16) * 256 + o * 16 + d % 16
            -> [page][head][dim chunk of 16][token][16 dims]
  V codes:  (p*H + h) * 4096 + d * 16 + o
            -> [page][head][dim][token]: the 16 tokens of one dim are one 16-byte run
            (the article's V cache [blocks, heads, head_dim, block_size], §2.3)
  K and V scales (fp32): (p*H + h) * 16 + o

These formulas are the library's published layout (its C header states the same
ones); this module evaluates them with NumPy fancy indexing only.
"""
from __future__ import annotations

import numpy as np

PAGE = 16
HEAD_DIM = 256
BLOCK_BYTES = PAGE * HEAD_DIM  # 4096 bytes of codes per (page, head)


def k_offset(p, h, o, d, n_kv_heads):
    p, h, o, d = (np.asarray(a, dtype=np.int64) for a in (p, h, o, d))
    return ((p * n_kv_heads + h) * 16 + d // 16) * 256 + o * 16 + d % 16


def v_offset(p, h, o, d, n_kv_heads):
    p, h, o, d = (np.asarray(a, dtype=np.int64) for a in (p, h, o, d))
    return (p * n_kv_heads + h) * BLOCK_BYTES + d * PAGE + o


def scale_index(p, h, o, n_kv_heads):
    p, h, o = (np.asarray(a, dtype=np.int64) for a in (p, h, o))
    return (p * n_kv_heads + h) * PAGE + o


def alloc_cache(num_pages: int, n_kv_heads: int, fill_code: int = 0, fill_scale: float = 0.0):
    """(k_cache int8, v_cache int8, k_scale fp32, v_scale fp32), flat arrays."""
    n = num_pages * n_kv_heads
    return (np.full(n * BLOCK_BYTES, fill_code, dtype=np.int8),
            np.full(n * BLOCK_BYTES, fill_code, dtype=np.int8),
            np.full(n * PAGE, fill_scale, dtype=np.float32),
            np.full(n * PAGE, fill_scale, dtype=np.float32))


def write_rows(cache, slots, k_codes, k_scales, v_codes, v_scales):
    """Scatter rows into the cache in place. k_codes [T, H, D]; scales [T, H]; slots [T].

    A negative slot skips its row. Later rows win when two rows share a slot.
    """
    k_cache, v_cache, k_scale, v_scale = cache
    slots = np.asarray(slots, dtype=np.int64)
    keep = np.nonzero(slots >= 0)[0]
    if keep.size == 0:
        return cache
    T, H, D = k_codes.shape
    assert D == HEAD_DIM
    p = (slots[keep] // PAGE)[:, None, None]
    o = (slots[keep] % PAGE)[:, None, None]
    h = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    k_cache[k_offset(p, h, o, d, H)] = k_codes[keep]
    v_cache[v_offset(p, h, o, d, H)] = v_codes[keep]
    k_scale[scale_index(p[..., 0], h[..., 0], o[..., 0], H)] = k_scales[keep]
    v_scale[scale_index(p[..., 0], h[..., 0], o[..., 0], H)] = v_scales[keep]
    return cache


def gather_seq(cache, block_table_row, ctx: int, n_kv_heads: int):
    """Logical (k_codes [ctx,H,D], k_scales [ctx,H], v_codes, v_scales) of one sequence."""
    k_cache, v_cache, k_scale, v_scale = cache
    t = np.arange(ctx, dtype=np.int64)
    p = np.asarray(block_table_row, dtype=np.int64)[t // PAGE][:, None, None]
    o = (t % PAGE)[:, None, None]
    h = np.arange(n_kv_heads)[None, :, None]
    d = np.arange(HEAD_DIM)[None, None, :]
    kc = k_cache[k_offset(p, h, o, d, n_kv_heads)]
    vc = v_cache[v_offset(p, h, o, d, n_kv_heads)]
    ks = k_scale[scale_index(p[..., 0], h[..., 0], o[..., 0], n_kv_heads)]
    vs = v_scale[scale_index(p[..., 0], h[..., 0], o[..., 0], n_kv_heads)]
    return kc, ks, vc, vs
