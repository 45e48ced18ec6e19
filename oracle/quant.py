"""Per-row symmetric int8 quantizer (oracle). Test infrastructure only.

Rule ("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §2.1): for a row x of
head_dim values, amax = max|x|, scale = amax / 127, q = clamp(round(x / scale),
-127, 127), x ~ q * scale. Granularity is one scale per (token, head) row (§2.1,
§2.2); K and V rows are quantized independently, Q rows the same way (§2.2).

Readings where the article leaves a step open:
  * every operation is IEEE fp32 (the scales are stored as FP32, §2.3): amax is the
    exact fp32 maximum, scale = fl32(amax / 127) and the quotient is fl32(x / scale),
    both true divisions (no reciprocal multiply);
  * round() is round-half-to-even (np.rint);
  * amax = 0 ("safe scale or all-zero output", §2.1): scale 0.0 and all codes 0; the
    same holds whenever fl32(amax/127) underflows to 0;
  * -128 is never produced (range [-127, 127], §2.1).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bf16 (8 significant bits), ties to even;
    returns the bf16 bit patterns (uint16). Evaluated as m * 2^e with 0.5 <= |m| < 1:
    rint(m * 2^8) / 2^8 is exact in float64, so the only rounding is rint's."""
    x = np.asarray(x, dtype=np.float32)
    m, e = np.frexp(x.astype(np.float64))
    r = np.ldexp(np.rint(m * 256.0) / 256.0, e).astype(np.float32)   # exact: <= 9 bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize the last axis of x (fp32). Returns (codes int8, scales fp32 [x.shape[:-1]])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)                       # exact in fp32
    scale = np.divide(amax, np.float32(127.0), dtype=np.float32)
    live = scale > 0
    safe = np.where(live, scale, np.float32(1.0)).astype(np.float32)
    quot = np.divide(x, safe[..., None], dtype=np.float32)  # fl32(x / scale)
    codes = np.clip(np.rint(quot), -127.0, 127.0)
    codes = np.where(live[..., None], codes, 0.0).astype(np.int8)
    return codes, scale.astype(np.float32)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes * scale in float64 (exact: an int8 times an fp32 fits in a double)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]
