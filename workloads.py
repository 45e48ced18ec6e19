"""Seeded synthetic inputs for the INT8-KV attention path.

This module is shared by the tests, the benchmark and the smoke check. Both the
HIP path and the CPU oracle consume the bytes it produces. It holds none of the
method's arithmetic: no quantization, no dequantization, no attention. It only
draws random numbers, rounds fp32 to bf16 (a storage conversion of the inputs),
and lays out slot mappings and block tables.

Shapes follow the full-attention geometry of the model the INT8 KV article
studies: 24 query heads over 4 KV heads at head_dim 256, in 16-token pages
("INT8 KV and INT8 MMAC attention on a gfx936 DCU", §1.1 and §2.3).

Recipe of a case (draw order matters and is fixed):
  1. context lengths (batched case only): log-uniform in [lo, hi];
  2. K outlier channels: `k_outliers` distinct channel indices;
  3. page permutation of the shared pool (or the identity);
  4. per sequence, from its own child generator: K fp32 N(0,1), then V fp32
     N(0,1), then Q fp32 N(0,1) rounded to bf16 (round half to even);
  5. K outlier channels are multiplied by 10 (same channels for every token and
     KV head).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np

HEAD_DIM = 256
N_Q_HEADS = 24
N_KV_HEADS = 4
PAGE = 16            # tokens per page
PARTITION = 512      # decode split-K partition (rows of KV per partition)
SM_SCALE = 1.0 / 16.0  # 1/sqrt(256), exact in fp32

# The five workloads the path is measured and checked on. Sizes are those of the
# model geometry above; seeds are fixed.
CONFIGS = {
    1: dict(kind="decode", seed=0, ctx=[256], pages="identity", k_outliers=0,
            name="decode ctx=256, 1 seq, identity pages"),
    2: dict(kind="decode", seed=1, ctx=[3328], pages="random", k_outliers=4,
            name="decode ctx=3328, 1 seq, random pages, 4 K outlier channels x10"),
    3: dict(kind="decode", seed=2, ctx=[32768], pages="random", k_outliers=0,
            name="decode ctx=32768, 1 seq, random pages"),
    4: dict(kind="prefill", seed=3, ctx=32768, n_new=2048, pages="random", k_outliers=4,
            name="causal prefill chunk: 2048 new queries at ctx=32768 (30720 cached), random pages"),
    5: dict(kind="decode", seed=4, n_seqs=64, ctx_range=(1024, 131072), pages="random",
            k_outliers=0, name="batched decode: 64 seqs, ctx log-uniform [1024,131072], shared pool"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    Inputs here are finite normals, so NaN handling is not needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + bias) >> 16).astype(np.uint16)


@dataclasses.dataclass
class DecodeCase:
    """One decode batch. K/V rows are listed sequence by sequence, token order."""
    seed: int
    context_lens: np.ndarray        # int32 [S]
    block_table: np.ndarray         # int32 [S, max_blocks]; padding entries are 0
    num_pages: int
    k_outlier_channels: np.ndarray  # int64 [n] (may be empty)
    n_q_heads: int = N_Q_HEADS
    n_kv_heads: int = N_KV_HEADS
    head_dim: int = HEAD_DIM
    q_rows_per_seq: int = 1         # query tokens per sequence (1 = decode)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.sum())

    def seq_rng(self, s: int) -> np.random.Generator:
        return np.random.default_rng([self.seed, 1000 + s])

    def seq_data(self, s: int):
        """(k fp32 [ctx,Hkv,D], v fp32 [ctx,Hkv,D], q bf16-bits [rows,Hq,D]) of sequence s."""
        ctx = int(self.context_lens[s])
        rng = self.seq_rng(s)
        shape = (ctx, self.n_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        q = rng.standard_normal((self.q_rows_per_seq, self.n_q_heads, self.head_dim),
                                dtype=np.float32)
        if self.k_outlier_channels.size:
            k[:, :, self.k_outlier_channels] *= np.float32(10.0)
        return k, v, f32_to_bf16_bits(q)

    def seq_slots(self, s: int) -> np.ndarray:
        """Slot (page*16 + offset) of every token of sequence s, int32 [ctx]."""
        ctx = int(self.context_lens[s])
        t = np.arange(ctx, dtype=np.int64)
        pages = self.block_table[s, t // PAGE].astype(np.int64)
        return (pages * PAGE + t % PAGE).astype(np.int32)

    def iter_seqs(self) -> Iterator[tuple[int, np.ndarray, np.ndarray, np.ndarray, np.ndarray]]:
        for s in range(self.num_seqs):
            k, v, q = self.seq_data(s)
            yield s, k, v, q, self.seq_slots(s)

    def all_data(self):
        """Concatenated (k, v, q, slots) over all sequences (small cases only)."""
        ks, vs, qs, sl = [], [], [], []
        for _, k, v, q, slots in self.iter_seqs():
            ks.append(k); vs.append(v); qs.append(q); sl.append(slots)
        return (np.concatenate(ks), np.concatenate(vs), np.stack(qs), np.concatenate(sl))


def _pages_needed(ctx_lens) -> np.ndarray:
    return (np.asarray(ctx_lens, dtype=np.int64) + PAGE - 1) // PAGE


def make_decode_case(seed: int, ctx_lens, *, pages: str = "random", k_outliers: int = 0,
                     extra_pages: int = 0, q_rows_per_seq: int = 1,
                     n_q_heads: int = N_Q_HEADS, n_kv_heads: int = N_KV_HEADS,
                     head_dim: int = HEAD_DIM, max_blocks: int | None = None) -> DecodeCase:
    """A batch of sequences drawing pages from one shared pool.

    pages="identity": sequence pages are consecutive in pool order;
    pages="random": the pool is a random permutation dealt out to the sequences
    (no page is shared by two sequences). `extra_pages` adds unused pool pages.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    if np.any(ctx < 1):
        raise ValueError("context lengths must be >= 1")
    outl = (rng.choice(head_dim, size=k_outliers, replace=False)
            if k_outliers else np.zeros(0, dtype=np.int64))
    nb = _pages_needed(ctx)
    total = int(nb.sum()) + extra_pages
    order = rng.permutation(total) if pages == "random" else np.arange(total)
    mb = int(nb.max()) if max_blocks is None else int(max_blocks)
    table = np.zeros((ctx.shape[0], mb), dtype=np.int32)
    off = 0
    for s, n in enumerate(nb):
        table[s, :n] = order[off:off + n]
        off += int(n)
    return DecodeCase(seed=seed, context_lens=ctx.astype(np.int32), block_table=table,
                      num_pages=total, k_outlier_channels=np.sort(outl),
                      n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                      q_rows_per_seq=q_rows_per_seq)


def log_uniform_ctx(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U(ln lo, ln hi))) clipped to [lo, hi]; the first draw of the seed."""
    rng = np.random.default_rng([seed, 7])
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)


def config_case(cfg: int):
    """The DecodeCase (configs 1, 2, 3, 5) or PrefillCase (config 4) of a config."""
    c = CONFIGS[cfg]
    if c["kind"] == "prefill":
        return make_prefill_case(c["seed"], c["ctx"], c["n_new"], pages=c["pages"],
                                 k_outliers=c["k_outliers"])
    if "ctx_range" in c:
        ctx = log_uniform_ctx(c["seed"], c["n_seqs"], *c["ctx_range"])
    else:
        ctx = c["ctx"]
    return make_decode_case(c["seed"], ctx, pages=c["pages"], k_outliers=c["k_outliers"])


@dataclasses.dataclass
class PrefillCase:
    """One sequence: ctx - n_new cached rows plus n_new new rows, queries = new rows."""
    seed: int
    context_len: int
    n_new: int
    block_table: np.ndarray         # int32 [ceil(ctx/16)]
    num_pages: int
    k_outlier_channels: np.ndarray
    n_q_heads: int = N_Q_HEADS
    n_kv_heads: int = N_KV_HEADS
    head_dim: int = HEAD_DIM

    def data(self):
        """(k fp32 [ctx,Hkv,D], v fp32 [ctx,Hkv,D], q bf16-bits [n_new,Hq,D], slots int32 [ctx])."""
        rng = np.random.default_rng([self.seed, 1000])
        shape = (self.context_len, self.n_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        q = rng.standard_normal((self.n_new, self.n_q_heads, self.head_dim), dtype=np.float32)
        if self.k_outlier_channels.size:
            k[:, :, self.k_outlier_channels] *= np.float32(10.0)
        t = np.arange(self.context_len, dtype=np.int64)
        slots = (self.block_table[t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)
        return k, v, f32_to_bf16_bits(q), slots


def make_prefill_case(seed: int, ctx: int, n_new: int, *, pages: str = "random",
                      k_outliers: int = 0, extra_pages: int = 0,
                      n_q_heads: int = N_Q_HEADS, n_kv_heads: int = N_KV_HEADS,
                      head_dim: int = HEAD_DIM) -> PrefillCase:
    if not (1 <= n_new <= ctx):
        raise ValueError("need 1 <= n_new <= ctx")
    rng = np.random.default_rng(seed)
    outl = (rng.choice(head_dim, size=k_outliers, replace=False)
            if k_outliers else np.zeros(0, dtype=np.int64))
    nb = (ctx + PAGE - 1) // PAGE
    total = nb + extra_pages
    order = rng.permutation(total) if pages == "random" else np.arange(total)
    return PrefillCase(seed=seed, context_len=ctx, n_new=n_new,
                       block_table=order[:nb].astype(np.int32), num_pages=total,
                       k_outlier_channels=np.sort(outl), n_q_heads=n_q_heads,
                       n_kv_heads=n_kv_heads, head_dim=head_dim)


def rope_table(max_pos: int, rotary_dim: int, theta: float = 10000.0) -> np.ndarray:
    """A caller's RoPE table cos_sin [max_pos, rotary_dim] fp32: for position p and pair
    i < rotary_dim/2, cos and sin of p * theta^(-2i/rotary_dim) (evaluated in float64,
    rounded to fp32), cos in the first half of the row, sin in the second."""
    half = rotary_dim // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / rotary_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclasses.dataclass
class ProducerCase:
    """One producer batch: T tokens of q/k/v rows, their positions and cache slots."""
    seed: int
    positions: np.ndarray    # int32 [T]
    slots: np.ndarray        # int32 [T] (negative: skipped)
    num_pages: int
    rotary_dim: int
    max_pos: int
    n_q_heads: int = N_Q_HEADS
    n_kv_heads: int = N_KV_HEADS
    head_dim: int = HEAD_DIM

    def data(self):
        """(q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D]) fp32 N(0,1), K with 4 outlier channels x10."""
        rng = np.random.default_rng([self.seed, 2000])
        T = self.positions.shape[0]
        q = rng.standard_normal((T, self.n_q_heads, self.head_dim), dtype=np.float32)
        k = rng.standard_normal((T, self.n_kv_heads, self.head_dim), dtype=np.float32)
        v = rng.standard_normal((T, self.n_kv_heads, self.head_dim), dtype=np.float32)
        outl = rng.choice(self.head_dim, size=4, replace=False)
        k[:, :, outl] *= np.float32(10.0)
        return q, k, v

    def table(self):
        return rope_table(self.max_pos, self.rotary_dim)


def make_producer_case(seed: int, n_tokens: int, *, start: int = 0, layout: str = "chunk",
                       rotary_dim: int = HEAD_DIM, extra_pages: int = 2) -> ProducerCase:
    """layout="chunk": tokens start..start+T-1 of one sequence at consecutive positions,
    written to a random permutation of pages (whole-page runs where the chunk covers a
    page); layout="scatter": T decode tokens of T sequences at random positions and random
    slots (one slot per token, some slots skipped with -1)."""
    rng = np.random.default_rng([seed, 2001])
    if layout == "chunk":
        pos = np.arange(start, start + n_tokens, dtype=np.int64)
        n_pages = int(pos[-1] // PAGE) + 1 + extra_pages
        perm = rng.permutation(n_pages)
        slots = perm[pos // PAGE] * PAGE + pos % PAGE
        max_pos = int(pos[-1]) + 1
    else:
        n_pages = n_tokens + extra_pages
        pos = rng.integers(0, 131072, size=n_tokens)
        slots = rng.permutation(n_pages * PAGE)[:n_tokens]
        slots[rng.random(n_tokens) < 0.1] = -1
        max_pos = 131072
    return ProducerCase(seed=seed, positions=pos.astype(np.int32), slots=slots.astype(np.int32),
                        num_pages=n_pages, rotary_dim=rotary_dim, max_pos=max_pos)


def near_tie_rows(seed: int, n_rows: int, head_dim: int = HEAD_DIM) -> np.ndarray:
    """fp32 rows built to sit on or next to rounding ties of x/scale.

    Each row has amax = 127*s for a random s, so scale = s up to rounding; the other
    elements are (k + 0.5)*s nudged by -1, 0 or +1 ulp. These are the inputs where
    a reciprocal-multiply or a wrong rounding mode gives a different code.
    """
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(-8.0, 4.0, size=(n_rows, 1))).astype(np.float32)
    kk = rng.integers(-127, 127, size=(n_rows, head_dim)).astype(np.float32)
    x = ((kk + np.float32(0.5)) * s).astype(np.float32)
    nudge = rng.integers(-1, 2, size=x.shape)
    x = np.where(nudge > 0, np.nextafter(x, np.float32(np.inf)),
                 np.where(nudge < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
    col = rng.integers(0, head_dim, size=n_rows)
    sign = np.where(rng.random(n_rows) < 0.5, -1.0, 1.0).astype(np.float32)
    x[np.arange(n_rows), col] = sign * np.float32(127.0) * s[:, 0]
    return x
