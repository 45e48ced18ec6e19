"""Python binding of libint8attn.so (MI355X / gfx950 INT8-KV paged attention).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. torch tensors supply device memory and the current HIP stream; nothing here
computes on the host and there is no fallback path: if the library is missing or a
call fails, an exception is raised.

The functions mirror the C ABI in include/int8attn.h (same names, same layout).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

__all__ = ["lib", "PagedCache", "alloc_cache", "kv_quant_write", "q_quant", "attn_decode",
           "attn_decode_workspace_bytes", "attn_verify", "attn_verify_workspace_bytes",
           "attn_decode_int8p", "attn_decode_int8p_workspace_bytes", "attn_decode_partition_rows",
           "attn_prefill_chunk", "attn_prefill_chunk_split",
           "attn_prefill_chunk_split_workspace_bytes", "kv_produce", "attn_chunk_bf16",
           "attn_chunk_bf16_workspace_bytes", "prefill_step",
           "prefill_step_workspace_bytes", "check_block_table", "check_slots", "ceiling_stream_read", "attn_decode_noalloc",
           "ceiling_mfma_i8", "ceiling_page_gather", "Int8AttnError",
           "HEAD_DIM", "PAGE", "PARTITION", "EXPORTED_SYMBOLS"]

HEAD_DIM = 256
PAGE = 16
PARTITION = 512
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint8attn.so")
EXPORTED_SYMBOLS = ("int8attn_last_error", "int8attn_version", "kv_quant_write", "kv_produce",
                    "q_quant", "attn_decode_q8", "attn_verify_q8", "attn_decode_int8p_q8",
                    "attn_prefill_chunk_q8", "attn_chunk_bf16", "prefill_step_workspace_bytes",
                    "prefill_step",
                    "attn_decode_workspace_bytes", "attn_decode", "attn_verify_workspace_bytes",
                    "attn_verify", "attn_decode_partition_rows",
                    "attn_decode_int8p_workspace_bytes", "attn_decode_int8p",
                    "attn_prefill_chunk", "attn_prefill_chunk_split_workspace_bytes",
                    "attn_prefill_chunk_split", "attn_prefill_chunk_split_q8",
                    "attn_chunk_bf16_workspace_bytes", "int8attn_check_block_table",
                    "int8attn_check_slots", "int8attn_ceiling_stream_read",
                    "int8attn_ceiling_mfma_i8", "int8attn_ceiling_mfma_i8_count",
                    "int8attn_ceiling_page_gather",
                    "attn_decode_noalloc", "attn_decode_noalloc_max_bytes")

_c_void = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t
_c_float = ctypes.c_float

_SIGNATURES = {
    "int8attn_last_error": (ctypes.c_char_p, []),
    "int8attn_version": (_c_int, []),
    "kv_quant_write": (_c_int, [_c_void, _c_void, _c_int, _c_int, _c_int, _c_int, _c_void,
                                _c_void, _c_void, _c_void, _c_void, _c_int, _c_void]),
    "kv_produce": (_c_int, [_c_void, _c_void, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_void, _c_void, _c_int, _c_int, _c_void, _c_void, _c_void, _c_void,
                            _c_void, _c_int, _c_void, _c_void, _c_void, _c_void, _c_void]),
    "attn_chunk_bf16": (_c_int, [_c_void, _c_void, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_float, _c_void, _c_void, _c_size, _c_void]),
    "attn_chunk_bf16_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "prefill_step_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "prefill_step": (_c_int, [_c_void, _c_void, _c_void, _c_int, _c_void, _c_void, _c_int, _c_int,
                              _c_void, _c_void, _c_void, _c_void, _c_void, _c_int, _c_void, _c_int,
                              _c_int, _c_int, _c_int, _c_float, _c_void, _c_void, _c_size,
                              _c_void]),
    "q_quant": (_c_int, [_c_void, _c_int, _c_int, _c_void, _c_void, _c_void]),
    "attn_decode_q8": (_c_int, [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_void,
                                _c_int, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_float, _c_void, _c_void, _c_size, _c_void]),
    "attn_verify_q8": (_c_int, [_c_void, _c_void, _c_int, _c_void, _c_void, _c_void, _c_void,
                                _c_void, _c_int, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, _c_float, _c_void, _c_void, _c_size, _c_void]),
    "attn_decode_int8p_q8": (_c_int, [_c_void, _c_void, _c_int, _c_void, _c_void, _c_void,
                                      _c_void, _c_void, _c_int, _c_void, _c_int, _c_int, _c_int,
                                      _c_int, _c_int, _c_int, _c_int, _c_float, _c_void, _c_void,
                                      _c_size, _c_void]),
    "attn_prefill_chunk_q8": (_c_int, [_c_void, _c_void, _c_int, _c_void, _c_void, _c_void,
                                       _c_void, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_float, _c_void, _c_void]),
    "attn_decode_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "attn_decode": (_c_int, [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_int,
                             _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                             _c_void, _c_void, _c_size, _c_void]),
    "attn_verify_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "attn_verify": (_c_int, [_c_void, _c_int, _c_void, _c_void, _c_void, _c_void, _c_void, _c_int,
                             _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                             _c_void, _c_void, _c_size, _c_void]),
    "attn_decode_partition_rows": (_c_int, [_c_int, _c_int, _c_int]),
    "attn_decode_int8p_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                    _c_int]),
    "attn_decode_int8p": (_c_int, [_c_void, _c_int, _c_void, _c_void, _c_void, _c_void, _c_void,
                                   _c_int, _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _c_float, _c_void, _c_void, _c_size, _c_void]),
    "attn_prefill_chunk": (_c_int, [_c_void, _c_int, _c_void, _c_void, _c_void, _c_void,
                                    _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_void, _c_void]),
    "attn_prefill_chunk_split_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int,
                                                           _c_int, _c_int]),
    "attn_prefill_chunk_split": (_c_int, [_c_void, _c_int, _c_void, _c_void, _c_void, _c_void,
                                          _c_void, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_float, _c_void, _c_void, _c_size, _c_void]),
    "int8attn_check_block_table": (_c_int, [_c_void, _c_int, _c_int, _c_void, _c_int, _c_int]),
    "int8attn_check_slots": (_c_int, [_c_void, _c_int, _c_int]),
    "attn_decode_noalloc_max_bytes": (_c_size, []),
    "attn_decode_noalloc": (_c_int, [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_int,
                                     _c_void, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_float, _c_void, _c_void]),
    "int8attn_ceiling_stream_read": (_c_int, [_c_void, _c_size, _c_void, _c_int, _c_void]),
    "int8attn_ceiling_mfma_i8": (_c_int, [_c_int, _c_int, _c_void, _c_void]),
    "int8attn_ceiling_mfma_i8_count": (ctypes.c_int64, [_c_int, _c_int]),
    "int8attn_ceiling_page_gather": (_c_int, [_c_void] * 5 + [_c_int] * 4 + [_c_void, _c_void]),
    "attn_prefill_chunk_split_q8": (_c_int, [_c_void, _c_void, _c_int, _c_void, _c_void,
                                             _c_void, _c_void, _c_void, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_float, _c_void, _c_void,
                                             _c_size, _c_void]),
}


class Int8AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"int8attn error {code}: {msg}")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libint8attn.so (built in-tree by int8_kv_cache_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m int8_kv_cache_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(rc: int) -> None:
    if rc != 0:
        raise Int8AttnError(rc, lib().int8attn_last_error().decode())


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, contiguous=True) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


@dataclasses.dataclass
class PagedCache:
    """The four device arrays of the paged INT8 cache (layout: include/int8attn.h)."""
    k_cache: torch.Tensor   # int8 [num_pages * n_kv_heads * 4096]
    v_cache: torch.Tensor   # int8 [num_pages * n_kv_heads * 4096]
    k_scale: torch.Tensor   # fp32 [num_pages * n_kv_heads * 16]
    v_scale: torch.Tensor   # fp32 [num_pages * n_kv_heads * 16]
    num_pages: int
    n_kv_heads: int

    def __post_init__(self):
        blk = self.num_pages * self.n_kv_heads
        for t, n, dt in ((self.k_cache, blk * PAGE * HEAD_DIM, torch.int8),
                         (self.v_cache, blk * PAGE * HEAD_DIM, torch.int8),
                         (self.k_scale, blk * PAGE, torch.float32),
                         (self.v_scale, blk * PAGE, torch.float32)):
            if t.numel() != n or t.dtype != dt or not t.is_contiguous():
                raise ValueError("cache arrays do not match num_pages / n_kv_heads")

    def ptrs(self):
        return (_dev(self.k_cache, "k_cache", torch.int8), _dev(self.v_cache, "v_cache", torch.int8),
                _dev(self.k_scale, "k_scale", torch.float32),
                _dev(self.v_scale, "v_scale", torch.float32))


def alloc_cache(num_pages: int, n_kv_heads: int, device="cuda") -> PagedCache:
    """Zero-filled paged cache of num_pages pages."""
    n = num_pages * n_kv_heads
    return PagedCache(torch.zeros(n * PAGE * HEAD_DIM, dtype=torch.int8, device=device),
                      torch.zeros(n * PAGE * HEAD_DIM, dtype=torch.int8, device=device),
                      torch.zeros(n * PAGE, dtype=torch.float32, device=device),
                      torch.zeros(n * PAGE, dtype=torch.float32, device=device),
                      num_pages, n_kv_heads)


def kv_quant_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, cache,
                   stream=None) -> None:
    """Quantize K/V rows [T, Hkv, 256] (fp32 or bf16) into the paged cache at their slots."""
    if k.dim() != 3 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must both be [T, Hkv, head_dim] of one dtype")
    T, H, D = k.shape
    dt = {torch.float32: 0, torch.bfloat16: 1}.get(k.dtype)
    if dt is None:
        raise TypeError("k/v must be float32 or bfloat16")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    if H != cache.n_kv_heads:
        raise ValueError("k/v head count differs from the cache")
    _check(lib().kv_quant_write(_dev(k, "k"), _dev(v, "v"), dt, T, H, D,
                                _dev(slot_mapping, "slot_mapping", torch.int32), *cache.ptrs(),
                                cache.num_pages, _stream(stream)))


def kv_produce(q, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
               cos_sin: torch.Tensor | None, slot_mapping: torch.Tensor, cache,
               rotary_dim: int | None = None, stream=None, rotated_bf16: bool = False):
    """Fused producer: RoPE on q [T, Hq, 256] and k [T, Hkv, 256] (fp32 or bf16, one dtype)
    from the table cos_sin [max_pos, rotary_dim] (cos half, then sin half), quantize q, k,
    v, write k/v into the paged cache at their slots. Returns (q_codes int8 [T, Hq, 256],
    q_scales fp32 [T, Hq]), or None when q is None; with rotated_bf16 it returns the
    rotated (q, k) rows in bf16 instead. rotary_dim defaults to the table width (0: none)."""
    if k.dim() != 3 or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must both be [T, Hkv, head_dim] of one dtype")
    T, H, D = k.shape
    dt = {torch.float32: 0, torch.bfloat16: 1}.get(k.dtype)
    if dt is None:
        raise TypeError("k/v must be float32 or bfloat16")
    if slot_mapping.shape != (T,) or positions.shape != (T,):
        raise ValueError("slot_mapping and positions must be [T]")
    if H != cache.n_kv_heads:
        raise ValueError("k/v head count differs from the cache")
    rd = (cos_sin.shape[1] if cos_sin is not None else 0) if rotary_dim is None else int(rotary_dim)
    max_pos = cos_sin.shape[0] if cos_sin is not None else 0
    cs = _dev(cos_sin, "cos_sin", torch.float32) if cos_sin is not None else None
    qr = kr = None
    cp = sp = qrp = krp = None
    if q is not None:
        if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D or q.dtype != k.dtype:
            raise ValueError("q must be [T, Hq, head_dim] of k's dtype")
        Hq = q.shape[1]
        qp = _dev(q, "q")
        if rotated_bf16:
            qr = torch.empty(q.shape, dtype=torch.bfloat16, device=k.device)
            kr = torch.empty(k.shape, dtype=torch.bfloat16, device=k.device)
            qrp, krp = qr.data_ptr(), kr.data_ptr()
        else:
            codes = torch.empty(q.shape, dtype=torch.int8, device=k.device)
            scales = torch.empty(q.shape[:2], dtype=torch.float32, device=k.device)
            cp, sp = codes.data_ptr(), scales.data_ptr()
    else:
        Hq, qp = 6 * H, None
    _check(lib().kv_produce(qp, _dev(k, "k"), _dev(v, "v"), dt, T, Hq, H, D,
                            _dev(positions, "positions", torch.int32), cs, rd, max_pos,
                            _dev(slot_mapping, "slot_mapping", torch.int32), *cache.ptrs(),
                            cache.num_pages, cp, sp, qrp, krp, _stream(stream)))
    if q is None:
        return None
    return (qr, kr) if rotated_bf16 else (codes, scales)


def attn_chunk_bf16_workspace_bytes(n: int, causal: bool, n_q_heads: int, n_kv_heads: int,
                                    head_dim: int = HEAD_DIM) -> int:
    return int(lib().attn_chunk_bf16_workspace_bytes(n, int(bool(causal)), n_q_heads, n_kv_heads,
                                                     head_dim))


def attn_chunk_bf16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                    sm_scale: float | None = None, out: torch.Tensor | None = None,
                    stream=None, workspace: torch.Tensor | None = None,
                    split: bool = True) -> torch.Tensor:
    """High-precision attention of a chunk over its own bf16 rows: q [n, Hq, 256],
    k/v [n, Hkv, 256] -> out fp32 [n, Hq, 256]. split: key partitions for causal chunks
    (a workspace is allocated when none is given); False: the one pass."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise TypeError(f"{nm} must be bfloat16 [n, heads, head_dim]")
    n, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != n:
        raise ValueError("k and v must be [n, Hkv, head_dim]")
    if out is None:
        out = torch.empty((n, Hq, D), dtype=torch.float32, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    ws_ptr, ws_bytes = None, 0
    if split:
        if workspace is None:
            need = attn_chunk_bf16_workspace_bytes(n, causal, Hq, k.shape[1], D)
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(lib().attn_chunk_bf16(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), n, int(bool(causal)),
                                 Hq, k.shape[1], D, sm, _dev(out, "out", torch.float32),
                                 ws_ptr, ws_bytes, _stream(stream)))
    return out


def prefill_step_workspace_bytes(n_new: int, context_len: int, n_q_heads: int, n_kv_heads: int,
                                 head_dim: int = HEAD_DIM) -> int:
    return int(lib().prefill_step_workspace_bytes(n_new, context_len, n_q_heads, n_kv_heads,
                                                  head_dim))


def prefill_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                 cos_sin: torch.Tensor, slot_mapping: torch.Tensor, cache,
                 block_table: torch.Tensor, context_len: int, sm_scale: float | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """One prefill chunk end to end (producer, then the route by history): q/k/v bf16 as
    projected [n_new, heads, 256] -> out fp32 [n_new, Hq, 256]."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise TypeError(f"{nm} must be bfloat16 [n_new, heads, head_dim]")
    n_new, Hq, D = q.shape
    if out is None:
        out = torch.empty((n_new, Hq, D), dtype=torch.float32, device=q.device)
    need = prefill_step_workspace_bytes(n_new, int(context_len), Hq, cache.n_kv_heads, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    _check(lib().prefill_step(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), n_new,
                              _dev(positions, "positions", torch.int32),
                              _dev(cos_sin, "cos_sin", torch.float32), cos_sin.shape[1],
                              cos_sin.shape[0], _dev(slot_mapping, "slot_mapping", torch.int32),
                              *cache.ptrs(), cache.num_pages,
                              _dev(block_table, "block_table", torch.int32), int(context_len),
                              Hq, cache.n_kv_heads, D, sm, _dev(out, "out", torch.float32),
                              _dev(workspace, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def _query(q: torch.Tensor, q_scales, dims: int, what: str):
    """bf16 rows (q_scales None) or int8 codes + fp32 scales of the same leading shape."""
    if q.dim() != dims:
        raise TypeError(f"q must have {dims} dims ({what})")
    if q_scales is None:
        if q.dtype != torch.bfloat16:
            raise TypeError("q must be bfloat16, or int8 codes with q_scales")
        return None
    if q.dtype != torch.int8 or q_scales.dtype != torch.float32 or q_scales.shape != q.shape[:-1]:
        raise TypeError("int8 q needs fp32 q_scales of shape q.shape[:-1]")
    return _dev(q_scales, "q_scales", torch.float32)


def q_quant(q: torch.Tensor, stream=None):
    """bf16 rows [..., 256] -> (int8 codes [..., 256], fp32 scales [...])."""
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    D = q.shape[-1]
    rows = q.numel() // D
    codes = torch.empty(q.shape, dtype=torch.int8, device=q.device)
    scales = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    _check(lib().q_quant(_dev(q, "q"), rows, D, codes.data_ptr(), scales.data_ptr(),
                         _stream(stream)))
    return codes, scales


def attn_decode_workspace_bytes(num_seqs: int, max_context_len: int, n_q_heads: int,
                                head_dim: int = HEAD_DIM) -> int:
    return int(lib().attn_decode_workspace_bytes(num_seqs, max_context_len, n_q_heads, head_dim))


def attn_decode(q: torch.Tensor, cache, block_table: torch.Tensor, context_lens: torch.Tensor,
                max_context_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None,
                q_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Decode: q bf16 [S, Hq, 256] (or int8 codes with q_scales [S, Hq]) -> out fp32
    [S, Hq, 256] over the paged INT8 cache."""
    qs = _query(q, q_scales, 3, "[S, Hq, head_dim]")
    S, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [S]")
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(S, max_context_len, Hq, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    fn, head = ((lib().attn_decode, (_dev(q, "q"),)) if qs is None
                else (lib().attn_decode_q8, (_dev(q, "q"), qs)))
    _check(fn(*head, *cache.ptrs(),
                             _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                             _dev(context_lens, "context_lens", torch.int32), S,
                             int(max_context_len), cache.num_pages, Hq, cache.n_kv_heads, D, sm,
                             _dev(out, "out", torch.float32), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def attn_verify_workspace_bytes(num_seqs: int, nq: int, max_context_len: int, n_q_heads: int,
                                head_dim: int = HEAD_DIM) -> int:
    return int(lib().attn_verify_workspace_bytes(num_seqs, nq, max_context_len, n_q_heads, head_dim))


def attn_verify(q: torch.Tensor, cache, block_table: torch.Tensor, context_lens: torch.Tensor,
                max_context_len: int, sm_scale: float | None = None, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None,
                q_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Multi-row decode: q bf16 [S, nq, Hq, 256] (or int8 codes with q_scales [S, nq, Hq];
    query i of a sequence at position ctx - nq + i) -> out fp32 [S, nq, Hq, 256]."""
    qs = _query(q, q_scales, 4, "[S, nq, Hq, head_dim]")
    S, nq, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [S]")
    if out is None:
        out = torch.empty((S, nq, Hq, D), dtype=torch.float32, device=q.device)
    need = attn_verify_workspace_bytes(S, nq, max_context_len, Hq, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    fn, head = ((lib().attn_verify, (_dev(q, "q"),)) if qs is None
                else (lib().attn_verify_q8, (_dev(q, "q"), qs)))
    _check(fn(*head, nq, *cache.ptrs(),
                             _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                             _dev(context_lens, "context_lens", torch.int32), S,
                             int(max_context_len), cache.num_pages, Hq, cache.n_kv_heads, D, sm,
                             _dev(out, "out", torch.float32), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def attn_decode_partition_rows(num_seqs: int, max_context_len: int, n_kv_heads: int) -> int:
    return int(lib().attn_decode_partition_rows(num_seqs, max_context_len, n_kv_heads))


def attn_decode_int8p_workspace_bytes(num_seqs: int, nq: int, max_context_len: int,
                                      n_q_heads: int, n_kv_heads: int, head_dim: int = HEAD_DIM,
                                      partition_rows: int = 0) -> int:
    return int(lib().attn_decode_int8p_workspace_bytes(num_seqs, nq, max_context_len, n_q_heads,
                                                       n_kv_heads, head_dim, partition_rows))


def attn_decode_int8p(q: torch.Tensor, cache, block_table: torch.Tensor,
                      context_lens: torch.Tensor, max_context_len: int, partition_rows: int = 0,
                      sm_scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None,
                      q_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Int8-P decode/verify: q bf16 [S, Hq, 256] (one row) or [S, nq, Hq, 256] (or int8
    codes with q_scales) -> out fp32 of the same shape."""
    qs = _query(q, q_scales, q.dim() if q.dim() in (3, 4) else 4, "[S, (nq,) Hq, head_dim]")
    one_row = q.dim() == 3
    q4 = q.unsqueeze(1) if one_row else q
    S, nq, Hq, D = q4.shape
    if block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("block_table must be [S, max_blocks]")
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [S]")
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    need = attn_decode_int8p_workspace_bytes(S, nq, max_context_len, Hq, cache.n_kv_heads, D,
                                             partition_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    fn, head = ((lib().attn_decode_int8p, (_dev(q4, "q"),)) if qs is None
                else (lib().attn_decode_int8p_q8, (_dev(q4, "q"), qs)))
    _check(fn(*head, nq, *cache.ptrs(),
                                   _dev(block_table, "block_table", torch.int32),
                                   block_table.shape[1],
                                   _dev(context_lens, "context_lens", torch.int32), S,
                                   int(max_context_len), cache.num_pages, Hq, cache.n_kv_heads, D,
                                   int(partition_rows), sm, _dev(out, "out", torch.float32),
                                   _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def attn_prefill_chunk(q: torch.Tensor, cache, block_table: torch.Tensor, context_len: int,
                       causal: bool = True, sm_scale: float | None = None,
                       out: torch.Tensor | None = None, stream=None,
                       q_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Chunk: q bf16 [n_new, Hq, 256] (or int8 codes with q_scales [n_new, Hq]) at the
    tail of one sequence -> out fp32 [n_new, Hq, 256]."""
    qs = _query(q, q_scales, 3, "[n_new, Hq, head_dim]")
    n_new, Hq, D = q.shape
    if block_table.dim() != 1 or block_table.numel() < (context_len + PAGE - 1) // PAGE:
        raise ValueError("block_table must be [ceil(context_len/16)]")
    if out is None:
        out = torch.empty((n_new, Hq, D), dtype=torch.float32, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    fn, head = ((lib().attn_prefill_chunk, (_dev(q, "q"),)) if qs is None
                else (lib().attn_prefill_chunk_q8, (_dev(q, "q"), qs)))
    _check(fn(*head, n_new, *cache.ptrs(),
                                    _dev(block_table, "block_table", torch.int32),
                                    int(context_len), int(bool(causal)), cache.num_pages, Hq,
                                    cache.n_kv_heads, D, sm,
                                    _dev(out, "out", torch.float32), _stream(stream)))
    return out


def attn_prefill_chunk_split_workspace_bytes(n_new: int, context_len: int, causal: bool,
                                             n_q_heads: int, n_kv_heads: int,
                                             head_dim: int = HEAD_DIM) -> int:
    return int(lib().attn_prefill_chunk_split_workspace_bytes(n_new, context_len, int(bool(causal)),
                                                              n_q_heads, n_kv_heads, head_dim))


def attn_prefill_chunk_split(q: torch.Tensor, cache, block_table: torch.Tensor, context_len: int,
                             causal: bool = True, sm_scale: float | None = None,
                             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             stream=None, q_scales: torch.Tensor | None = None) -> torch.Tensor:
    """attn_prefill_chunk with the keys split over workgroups for short causal chunks
    (a merge kernel combines the partitions); other chunks take the one pass."""
    qs = _query(q, q_scales, 3, "[n_new, Hq, head_dim]")
    n_new, Hq, D = q.shape
    if block_table.dim() != 1 or block_table.numel() < (context_len + PAGE - 1) // PAGE:
        raise ValueError("block_table must be [ceil(context_len/16)]")
    if out is None:
        out = torch.empty((n_new, Hq, D), dtype=torch.float32, device=q.device)
    need = attn_prefill_chunk_split_workspace_bytes(n_new, context_len, causal, Hq,
                                                    cache.n_kv_heads, D)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    fn, head = ((lib().attn_prefill_chunk_split, (_dev(q, "q"),)) if qs is None
                else (lib().attn_prefill_chunk_split_q8, (_dev(q, "q"), qs)))
    _check(fn(*head, n_new, *cache.ptrs(), _dev(block_table, "block_table", torch.int32),
              int(context_len), int(bool(causal)), cache.num_pages, Hq, cache.n_kv_heads, D, sm,
              _dev(out, "out", torch.float32), _dev(workspace, "workspace"),
              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def _host_i32(a, name: str):
    """A host int32 contiguous copy of a numpy array or torch tensor (any device)."""
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().to("cpu").numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"{name} must be int32, got {a.dtype}")
    return a


def check_block_table(block_table, context_lens, max_context_len: int, num_pages: int) -> None:
    """Opt-in check of paging metadata (int8attn_check_block_table on host copies):
    block_table [S, max_blocks] with context_lens [S], or a single table row [blocks] with
    context_lens None (one sequence of max_context_len keys, as attn_prefill_chunk takes).
    Raises Int8AttnError naming the first entry outside the pool or bad context length."""
    t = _host_i32(block_table, "block_table")
    if t.ndim == 1:
        t = t[None, :]
    if t.ndim != 2:
        raise ValueError("block_table must be [S, max_blocks] or [blocks]")
    c = None if context_lens is None else _host_i32(context_lens, "context_lens")
    if c is not None and c.shape != (t.shape[0],):
        raise ValueError("context_lens must be [S]")
    _check(lib().int8attn_check_block_table(t.ctypes.data, t.shape[0], t.shape[1],
                                            None if c is None else c.ctypes.data,
                                            int(max_context_len), int(num_pages)))


def check_slots(slot_mapping, num_pages: int) -> None:
    """Opt-in check of a writer's slot_mapping [T] (int8attn_check_slots on a host copy):
    raises Int8AttnError for a slot outside the pool or one named by two tokens."""
    s = _host_i32(slot_mapping, "slot_mapping").reshape(-1)
    _check(lib().int8attn_check_slots(s.ctypes.data, s.shape[0], int(num_pages)))


def ceiling_stream_read(src: torch.Tensor, n_workgroups: int, sink: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Measurement kernel: one 16-byte-load pass over src's bytes (the measured read
    ceiling); returns the sink [4 * n_workgroups] uint32 (as int32)."""
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(4 * n_workgroups, dtype=torch.int32, device=src.device)
    if sink.numel() < 4 * n_workgroups:
        raise ValueError("sink needs 4 words per workgroup")
    _check(lib().int8attn_ceiling_stream_read(_dev(src, "src"), nbytes, _dev(sink, "sink"),
                                              int(n_workgroups), _stream(stream)))
    return sink


def ceiling_page_gather(cache, block_table: torch.Tensor, n_blocks: int,
                        pages_per_workgroup: int, sink: torch.Tensor, stream=None) -> int:
    """Measurement kernel: the decode's reads (K and V codes and scales of the first n_blocks
    pages of a block-table row, every KV head) without its arithmetic; returns the bytes
    read."""
    n_kv = cache.n_kv_heads
    nx = -(-int(n_blocks) // int(pages_per_workgroup))
    if sink.numel() < 4 * nx * n_kv:
        raise ValueError("sink needs 4 words per workgroup")
    _check(lib().int8attn_ceiling_page_gather(
        *cache.ptrs(), _dev(block_table, "block_table", torch.int32), int(n_blocks), n_kv,
        int(cache.num_pages), int(pages_per_workgroup), _dev(sink, "sink"), _stream(stream)))
    return int(n_blocks) * (n_kv * (2 * 4096 + 2 * 64) + 4)


def ceiling_mfma_i8(n_workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> int:
    """Measurement kernel: a known number of int8 MFMAs (returned) on register operands."""
    if sink.numel() < n_workgroups:
        raise ValueError("sink needs one word per workgroup")
    _check(lib().int8attn_ceiling_mfma_i8(int(n_workgroups), int(iters), _dev(sink, "sink"),
                                          _stream(stream)))
    return int(lib().int8attn_ceiling_mfma_i8_count(int(n_workgroups), int(iters)))


def attn_decode_noalloc(q: torch.Tensor, cache, block_table: torch.Tensor,
                        context_lens: torch.Tensor, max_context_len: int, out: torch.Tensor,
                        sm_scale: float | None = None, stream=None) -> torch.Tensor:
    """attn_decode without a workspace (the library's fixed per-GPU scratch array holds the
    partials); `out` [S, Hq, 256] fp32 must be given, so nothing is allocated here either."""
    if q.dim() != 3 or q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16 [S, Hq, head_dim]")
    S, Hq, D = q.shape
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S, max_blocks] and context_lens [S]")
    if out.shape != (S, Hq, D):
        raise ValueError("out must be [S, Hq, head_dim]")
    sm = float(sm_scale if sm_scale is not None else D ** -0.5)
    _check(lib().attn_decode_noalloc(_dev(q, "q"), *cache.ptrs(),
                                     _dev(block_table, "block_table", torch.int32),
                                     block_table.shape[1],
                                     _dev(context_lens, "context_lens", torch.int32), S,
                                     int(max_context_len), cache.num_pages, Hq, cache.n_kv_heads,
                                     D, sm, _dev(out, "out", torch.float32), _stream(stream)))
    return out
