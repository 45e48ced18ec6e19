"""The C-ABI library loads and exports every symbol the header declares; host-side
argument validation returns the documented error codes without enqueuing anything
(no GPU is touched: every call below fails validation before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import int8_kv_cache_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8attn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def _codes():
    src = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(I8A_\w+)\s+(-?\d+)", src)}


def test_header_declares_the_binding_symbols():
    assert _declared_functions() == sorted(m.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = m.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(_declared_functions()) <= exported


def test_version():
    assert m.lib().int8attn_version() >> 16 == 1


FAKE = 0x1000  # never dereferenced: every call below is rejected on the host


def _err(rc):
    return rc, m.lib().int8attn_last_error().decode()


def test_kv_quant_write_validation():
    C = _codes()
    L = m.lib()
    args = dict(k=FAKE, v=FAKE, dt=0, T=4, H=4, D=256, slots=FAKE, kc=FAKE, vc=FAKE, ks=FAKE,
                vs=FAKE, P=8, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return _err(L.kv_quant_write(a["k"], a["v"], a["dt"], a["T"], a["H"], a["D"], a["slots"],
                                     a["kc"], a["vc"], a["ks"], a["vs"], a["P"], a["s"]))

    assert call(dt=7)[0] == C["I8A_EINVAL"]
    assert call(D=128)[0] == C["I8A_EUNSUPPORTED"]
    assert call(T=-1)[0] == C["I8A_EINVAL"]
    assert call(P=0)[0] == C["I8A_EINVAL"]
    rc, msg = call(k=None)
    assert rc == C["I8A_EINVAL"] and "null" in msg
    assert call(T=0)[0] == C["I8A_OK"]          # empty input: no-op


def test_q_quant_validation():
    C = _codes()
    L = m.lib()
    assert L.q_quant(FAKE, 3, 64, FAKE, FAKE, None) == C["I8A_EUNSUPPORTED"]
    assert L.q_quant(None, 3, 256, FAKE, FAKE, None) == C["I8A_EINVAL"]
    assert L.q_quant(FAKE, 0, 256, FAKE, FAKE, None) == C["I8A_OK"]


def test_workspace_bytes_formula():
    L = m.lib()
    # num_seqs * n_q_heads * ceil(ctx/512) * (2 + 256) floats, rounded up to 256 bytes
    assert L.attn_decode_workspace_bytes(1, 32768, 24, 256) == 24 * 64 * 258 * 4
    assert L.attn_decode_workspace_bytes(3, 513, 24, 256) == ((3 * 24 * 2 * 258 * 4 + 255) // 256) * 256
    assert L.attn_decode_workspace_bytes(0, 512, 24, 256) == 0
    assert L.attn_decode_workspace_bytes(1, 512, 24, 128) == 0


def test_attn_decode_validation():
    C = _codes()
    L = m.lib()
    base = [FAKE] * 6 + [16, FAKE, 1, 256, 16, 24, 4, 256, 0.0625, FAKE, FAKE, 10 ** 7, None]

    def call(i=None, val=None):
        a = list(base)
        if i is not None:
            a[i] = val
        return L.attn_decode(*a)

    assert call(12, 8) == C["I8A_EUNSUPPORTED"]        # 24 q heads over 8 kv heads
    assert call(13, 128) == C["I8A_EUNSUPPORTED"]      # head_dim
    a = list(base)
    a[11], a[12] = 6 * 11000, 11000                    # query heads beyond the merge grid
    assert L.attn_decode(*a) == C["I8A_EINVAL"]
    assert call(9, 0) == C["I8A_EINVAL"]               # max_context_len
    assert call(10, 0) == C["I8A_EINVAL"]              # num_pages
    assert call(14, float("nan")) == C["I8A_EINVAL"]   # sm_scale
    assert call(0, None) == C["I8A_EINVAL"]            # q null
    assert call(17, 100) == C["I8A_EWORKSPACE"]
    assert call(16, FAKE + 4) == C["I8A_EINVAL"]       # misaligned workspace
    assert call(8, 0) == C["I8A_OK"]                   # no sequences: no-op


def test_attn_verify_validation():
    C = _codes()
    L = m.lib()
    ws = m.attn_verify_workspace_bytes(2, 4, 1000, 24)
    assert ws == m.attn_decode_workspace_bytes(8, 1000, 24)
    assert m.attn_verify_workspace_bytes(2, 1, 1000, 24) == m.attn_decode_workspace_bytes(2, 1000, 24)
    assert m.attn_verify_workspace_bytes(2, 9, 1000, 24) == 0
    base = [FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 63, FAKE, 2, 1000, 200, 24, 4, 256, 0.0625,
            FAKE, FAKE, ws, None]

    def call(i=None, val=None):
        a = list(base)
        if i is not None:
            a[i] = val
        return L.attn_verify(*a)

    assert call(1, 0) == C["I8A_EINVAL"]                # nq < 1
    assert call(1, 9) == C["I8A_EINVAL"]                # nq > 8
    assert call(9, 20000) == C["I8A_EINVAL"]            # num_seqs * nq > 65535
    assert call(12, 12) == C["I8A_EUNSUPPORTED"]        # 12 q heads over 4 kv heads
    assert call(18, ws - 1) == C["I8A_EWORKSPACE"]
    assert call(16, None) == C["I8A_EINVAL"]            # out null
    assert call(9, 0) == C["I8A_OK"]                    # no sequences: no-op


def test_partition_law():
    law = m.attn_decode_partition_rows
    assert law(1, 256, 4) == 512        # one partition: no merge stage
    assert law(1, 512, 4) == 512
    assert law(1, 32768, 4) == 512      # 4 x 64 = 256 workgroups
    assert law(1, 8192, 4) == 512       # 4 x 16 = 64
    assert law(1, 4096, 4) == 256       # 4 x 8 = 32 -> 4 x 16 = 64
    assert law(1, 3328, 4) == 128       # 28 -> 52 -> 104
    assert law(1, 600, 4) == 128        # the 128-key floor
    assert law(64, 1024, 4) == 512
    assert law(0, 100, 4) == 0 and law(1, 0, 4) == 0


def test_attn_decode_int8p_validation():
    C = _codes()
    L = m.lib()
    ws = m.attn_decode_int8p_workspace_bytes(2, 1, 1000, 24, 4, partition_rows=64)
    assert ws == m.attn_decode_workspace_bytes(2, 1000 * 8, 24)   # 16 partials of 64 keys
    assert m.attn_decode_int8p_workspace_bytes(2, 1, 1000, 24, 4, partition_rows=0) == \
        m.attn_decode_workspace_bytes(2, 1000 * 4, 24)            # law: 128 (8 partials)
    assert m.attn_decode_int8p_workspace_bytes(2, 1, 1000, 24, 4, partition_rows=96) == 0
    base = [FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 63, FAKE, 2, 1000, 200, 24, 4, 256, 64, 0.0625,
            FAKE, FAKE, ws, None]

    def call(i=None, val=None):
        a = list(base)
        if i is not None:
            a[i] = val
        return L.attn_decode_int8p(*a)

    assert call(15, 96) == C["I8A_EINVAL"]              # partition size not in the list
    assert call(1, 9) == C["I8A_EINVAL"]                # nq > 8
    assert call(12, 18) == C["I8A_EUNSUPPORTED"]        # GQA group of 4.5
    assert call(19, ws - 1) == C["I8A_EWORKSPACE"]
    assert call(9, 0) == C["I8A_OK"]


def test_kv_produce_and_q8_validation():
    C = _codes()
    L = m.lib()
    base = [FAKE, FAKE, FAKE, 1, 4, 24, 4, 256, FAKE, FAKE, 64, 100, FAKE, FAKE, FAKE, FAKE, FAKE,
            10, FAKE, FAKE, None, None, None]

    def call(i=None, val=None):
        a = list(base)
        if i is not None:
            a[i] = val
        return L.kv_produce(*a)

    assert call(10, 12) == C["I8A_EINVAL"]              # rotary_dim not a multiple of 8
    assert call(10, 264) == C["I8A_EINVAL"]             # rotary_dim > head_dim
    assert call(9, None) == C["I8A_EINVAL"]             # RoPE without a table
    assert call(11, 0) == C["I8A_EINVAL"]               # ... or without positions range
    assert call(18, None) == C["I8A_EINVAL"]            # q_codes without q_scales
    assert call(5, 12) == C["I8A_EUNSUPPORTED"]         # group of 3
    assert call(3, 7) == C["I8A_EINVAL"]                # dtype
    assert call(4, 0) == C["I8A_OK"]                    # no tokens
    assert call(0, None) == C["I8A_EINVAL"]             # q_codes without q
    cb = [FAKE, FAKE, FAKE, 64, 2, 24, 4, 256, 0.0625, FAKE, None, 0, None]
    assert L.attn_chunk_bf16(*cb) == C["I8A_EINVAL"]    # causal flag
    # bf16 chunk split: 2,048 causal rows = 1,056 key blocks per KV head over 64 tiles;
    # x 4 heads / 256 CUs -> 17 blocks per CU, partitions of 17 * 6 / 5 = 20 blocks,
    # 2 partitions, rows 1,280.. merged
    cws = m.attn_chunk_bf16_workspace_bytes
    assert cws(2048, True, 24, 4) == (2048 - 1280) * 24 * 2 * 258 * 4
    assert cws(2048, False, 24, 4) == 0                 # non-causal: one pass
    assert cws(64, True, 24, 4) == 0                    # one key block
    # 3,000 rows: 2,256 blocks per head -> 36 per CU, partitions of 43 blocks (2,752 keys),
    # 2 partitions over the 47 blocks, rows 2,752.. merged; 6,000 rows: 188 tiles x 4 heads
    # keep the CUs busy and the plan keeps the one pass
    assert cws(3000, True, 24, 4) == (3000 - 43 * 64) * 24 * 2 * 258 * 4
    assert cws(6000, True, 24, 4) == 0
    need = cws(2048, True, 24, 4)
    cb = [FAKE, FAKE, FAKE, 2048, 1, 24, 4, 256, 0.0625, FAKE, FAKE, need - 1, None]
    assert L.attn_chunk_bf16(*cb) == C["I8A_EWORKSPACE"]
    cb[10], cb[11] = FAKE + 4, need
    assert L.attn_chunk_bf16(*cb) == C["I8A_EINVAL"]    # workspace not 16-byte aligned
    ps = m.prefill_step_workspace_bytes(100, 100, 24, 4)   # no history: rotated bf16 Q, K
    assert ps == (100 * 28 * 256 * 2 + 255) // 256 * 256 + m.attn_chunk_bf16_workspace_bytes(100, True, 24, 4)
    q8 = (100 * 24 * 260 + 255) // 256 * 256               # history: Q codes + split scratch
    assert m.prefill_step_workspace_bytes(100, 5000, 24, 4) == \
        q8 + m.attn_prefill_chunk_split_workspace_bytes(100, 5000, True, 24, 4)
    assert m.prefill_step_workspace_bytes(2048, 32768, 24, 4) == (2048 * 24 * 260 + 255) // 256 * 256
    step = [FAKE, FAKE, FAKE, 100, FAKE, FAKE, 64, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, 50, FAKE,
            100, 24, 4, 256, 0.0625, FAKE, 4096, ps - 1, None]
    assert L.prefill_step(*step) == C["I8A_EWORKSPACE"]
    dec = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 100, 10, 24, 4, 256, 0.0625,
           FAKE, FAKE, 1 << 20, None]
    assert L.attn_decode_q8(*dec) == C["I8A_EINVAL"]     # codes without scales
    pf = [FAKE, None, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24, 4, 256, 0.0625, FAKE, None]
    assert L.attn_prefill_chunk_q8(*pf) == C["I8A_EINVAL"]


def test_attn_prefill_validation():
    C = _codes()
    L = m.lib()
    base = [FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24, 4, 256, 0.0625, FAKE, None]

    def call(i=None, val=None):
        a = list(base)
        if i is not None:
            a[i] = val
        return L.attn_prefill_chunk(*a)

    assert call(10, 12) == C["I8A_EUNSUPPORTED"]
    assert call(11, 2**30) == C["I8A_EUNSUPPORTED"]    # 6 x n_kv_heads would overflow
    assert call(1, 101) == C["I8A_EINVAL"]             # n_new > context_len
    assert call(8, 2) == C["I8A_EINVAL"]               # causal flag
    assert call(7, 0) == C["I8A_EINVAL"]               # empty context
    assert call(14, None) == C["I8A_EINVAL"]           # out null
    assert call(9, 1 << 26) == C["I8A_EUNSUPPORTED"]   # pool past the 32-bit scale index
    assert call(1, 0) == C["I8A_OK"]                   # no queries: no-op


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        m.q_quant(torch.zeros(2, 256, dtype=torch.bfloat16))


def test_attn_prefill_split_workspace_and_validation():
    C = _codes()
    L = m.lib()
    wsb = m.attn_prefill_chunk_split_workspace_bytes
    assert wsb(200, 1500, False, 24, 4) == 0      # non-causal: the one pass
    assert wsb(1100, 5000, True, 24, 4) == 0      # 35 query blocks x 4 heads >= 128
    assert wsb(10, 64, True, 24, 4) == 0          # a single 64-key block
    assert wsb(0, 100, True, 24, 4) == 0
    assert wsb(16, 100, True, 24, 5) == 0         # not a group of 6
    assert wsb(16, 2**31 - 1, True, 24, 4) == 0   # context past the supported range
    assert wsb(16, 100, True, 24, 2**30) == 0     # head counts that would overflow
    assert m.prefill_step_workspace_bytes(16, 2**31 - 1, 24, 4) == 0
    up = lambda x: (x + 255) // 256 * 256

    def expect(rows, parts):
        # floats o[256], m and l per (row, head, partition), rounded up to 256 bytes; then
        # the query codes and scales, each rounded up to 256 bytes.
        return up(rows * parts * 258 * 4) + up(rows * 256) + up(rows * 4)

    # 16 rows, 100 keys = two 64-key blocks: 4 workgroups ask for 64 partitions, capped
    # at one block each = 2 partitions.
    assert wsb(16, 100, True, 24, 4) == expect(16 * 24, 2)
    # 12 rows at 20000 keys with one KV head: 256 partitions of 2 blocks -> 157 partitions
    assert wsb(12, 20000, True, 6, 1) == expect(12 * 6, 157)
    # At most 8 rows: the int8-P decode kernel's partials (m, l, o[256] per row, head and
    # partition of 256 keys here: 1 x 1 x 79 partitions of 256 reach 64 workgroups).
    assert wsb(3, 20000, True, 6, 1) == up(3 * 6 * 79 * 258 * 4)
    assert wsb(8, 32768, True, 24, 4) == up(8 * 24 * 64 * 258 * 4)  # 512-key partitions

    need = wsb(16, 100, True, 24, 4)
    base = [FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24, 4, 256, 0.0625, FAKE,
            FAKE, need, None]

    def call(i=None, val=None, fn=L.attn_prefill_chunk_split, args=base):
        a = list(args)
        if i is not None:
            a[i] = val
        return fn(*a)

    assert call(16, need - 1) == C["I8A_EWORKSPACE"]
    assert call(15, None) == C["I8A_EINVAL"]              # no workspace
    assert call(15, FAKE + 4) == C["I8A_EINVAL"]          # not 16-byte aligned
    assert call(8, 2) == C["I8A_EINVAL"]                  # causal flag
    assert call(10, 12) == C["I8A_EUNSUPPORTED"]
    assert call(1, 0) == C["I8A_OK"]                      # no queries: no-op
    # A chunk that takes the one pass needs no workspace.
    one = [FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 0, 16, 24, 4, 256, 0.0625, None,
           None, 0, None]
    assert call(fn=L.attn_prefill_chunk_split, args=one) == C["I8A_EINVAL"]  # (out null)
    q8 = [FAKE, None] + base[1:]
    assert call(fn=L.attn_prefill_chunk_split_q8, args=q8) == C["I8A_EINVAL"]  # no q_scales


def test_negative_sm_scale_is_refused_on_every_route():
    # The chunk kernel bounds its running max through the sign of the scale, so every
    # attention entry point refuses a negative (or non-finite) scale alike.
    C = _codes()
    L = m.lib()
    dec = [FAKE] * 6 + [16, FAKE, 1, 256, 16, 24, 4, 256, -0.0625, FAKE, FAKE, 10 ** 7, None]
    ver = [FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 63, FAKE, 2, 1000, 200, 24, 4, 256, -0.0625,
           FAKE, FAKE, 10 ** 8, None]
    i8p = [FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 63, FAKE, 2, 1000, 200, 24, 4, 256, 0, -0.0625,
           FAKE, FAKE, 10 ** 8, None]
    pf = [FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24, 4, 256, -0.0625, FAKE, None]
    sp = [FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24, 4, 256, -0.0625, FAKE,
          FAKE, 10 ** 8, None]
    cb = [FAKE, FAKE, FAKE, 64, 1, 24, 4, 256, -0.0625, FAKE, None, 0, None]
    step = [FAKE, FAKE, FAKE, 100, FAKE, FAKE, 64, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, 50, FAKE,
            100, 24, 4, 256, -0.0625, FAKE, 4096, 10 ** 8, None]
    for fn, a in ((L.attn_decode, dec), (L.attn_verify, ver), (L.attn_decode_int8p, i8p),
                  (L.attn_prefill_chunk, pf), (L.attn_prefill_chunk_split, sp),
                  (L.attn_chunk_bf16, cb), (L.prefill_step, step)):
        rc, msg = _err(fn(*a))
        assert rc == C["I8A_EINVAL"] and "sm_scale" in msg, (fn.__name__, rc, msg)
    # zero is allowed (uniform weights): it gets past the scale check to the null-pointer
    # check of the missing output
    a = list(pf)
    a[13], a[14] = 0.0, None
    rc, msg = _err(L.attn_prefill_chunk(*a))
    assert rc == C["I8A_EINVAL"] and "null" in msg


def test_check_block_table_names_the_first_bad_entry():
    import numpy as np
    C = _codes()
    table = np.array([[3, 1, 0, 0], [2, 4, 5, 0]], np.int32)
    ctx = np.array([20, 40], np.int32)               # 2 and 3 blocks used
    m.check_block_table(table, ctx, 64, 6)          # every used entry in [0, 6)
    m.check_block_table(table, np.array([0, 40], np.int32), 64, 6)   # context 0 is a padded slot
    bad = table.copy()
    bad[1, 2] = 6                                     # out of a pool of 6 pages
    with pytest.raises(m.Int8AttnError) as e:
        m.check_block_table(bad, ctx, 64, 6)
    assert e.value.code == C["I8A_EINVAL"]
    assert "sequence 1 block 2" in str(e.value) and "page 6" in str(e.value)
    bad[1, 2] = -1
    with pytest.raises(m.Int8AttnError, match="page -1"):
        m.check_block_table(bad, ctx, 64, 6)
    # an entry past the context is never read and not checked
    bad = table.copy()
    bad[0, 3] = 99
    m.check_block_table(bad, ctx, 64, 6)
    for c, why in (([20, 65], "above the table's 4 blocks"), ([20, -1], "negative"),
                   ([20, 40], "above max_context_len")):
        mc = 30 if why.endswith("max_context_len") else 64
        with pytest.raises(m.Int8AttnError, match="context"):
            m.check_block_table(table, np.array(c, np.int32), mc, 6)
    # one table row for a chunk: context_lens None = one sequence of max_context_len keys
    m.check_block_table(np.array([5, 0, 2], np.int32), None, 40, 6)
    with pytest.raises(m.Int8AttnError, match="block 2"):
        m.check_block_table(np.array([5, 0, 7], np.int32), None, 40, 6)
    L = m.lib()
    assert L.int8attn_check_block_table(None, 1, 4, None, 10, 6) == C["I8A_EINVAL"]
    assert L.int8attn_check_block_table(None, 0, 4, None, 10, 6) == C["I8A_OK"]
    assert L.int8attn_check_block_table(None, 1, 0, None, 10, 6) == C["I8A_EINVAL"]


def test_check_slots():
    import numpy as np
    C = _codes()
    m.check_slots(np.array([0, 17, -1, 95, -5], np.int32), 6)   # pool of 96 slots
    with pytest.raises(m.Int8AttnError, match="token 2 has slot 96"):
        m.check_slots(np.array([0, 17, 96], np.int32), 6)
    with pytest.raises(m.Int8AttnError, match="slot 17 is named by two tokens"):
        m.check_slots(np.array([17, 3, -1, -1, 17], np.int32), 6)
    with pytest.raises(TypeError):
        m.check_slots(np.array([1, 2], np.int64), 6)
    L = m.lib()
    assert L.int8attn_check_slots(None, 3, 6) == C["I8A_EINVAL"]
    assert L.int8attn_check_slots(None, 0, 6) == C["I8A_OK"]


def test_attn_decode_noalloc_limits_on_the_host():
    # the size check comes before any HIP call, so it runs without a GPU
    C = _codes()
    L = m.lib()
    assert m.lib().attn_decode_noalloc_max_bytes() == 32 << 20
    base = [FAKE] * 6 + [2048, FAKE, 22, 32768, 2048, 24, 4, 256, 0.0625, FAKE, None]
    rc, msg = _err(L.attn_decode_noalloc(*base))      # 22 x 24 x 64 x 1032 B > 32 MiB
    assert rc == C["I8A_EWORKSPACE"] and "attn_decode" in msg
    a = list(base)
    a[8] = 0
    assert L.attn_decode_noalloc(*a) == C["I8A_OK"]   # no sequences: no-op


def test_reciprocal_code_tie_band():
    # The kernels take each code as rint(x r), r the hardware reciprocal of the scale
    # (within one ulp of 1 / scale), rounding the exact product x r once (an fma onto
    # 1.5 * 2^23), unless x r lies within 2^-14 of a half-integer, where they use the IEEE
    # quotient x / scale. Checked here in numpy for reciprocals one ulp below, at and one
    # ulp above the correctly rounded one: every element whose code from x r differs from
    # rint(x / scale) lies inside that band, on rows built to sit on and next to rounding
    # ties at scales across the normal range.
    import numpy as np
    rng = np.random.default_rng(23)
    n_rows = 3000
    e = rng.integers(-125, 121, n_rows)
    amax = (np.ldexp(1.0 + rng.random(n_rows), e) * 127.0).astype(np.float32)
    rows = (rng.uniform(-1.0, 1.0, (n_rows, 256)) * amax[:, None]).astype(np.float32)
    sc = (amax / np.float32(127.0)).astype(np.float32)
    kk = rng.integers(-126, 126, rows.shape).astype(np.float32)
    tie = ((kk + np.float32(0.5)) * sc[:, None]).astype(np.float32)
    nudge = rng.integers(-1, 2, rows.shape)
    tie = np.where(nudge > 0, np.nextafter(tie, np.float32(np.inf)),
                   np.where(nudge < 0, np.nextafter(tie, np.float32(-np.inf)), tie)).astype(np.float32)
    keep = (np.abs(tie) < amax[:, None]) & (rng.random(rows.shape) < 0.5)
    rows[keep] = tie[keep]
    rows[np.arange(n_rows), rng.integers(0, 256, n_rows)] = amax
    scale = (np.abs(rows).max(axis=1) / np.float32(127.0)).astype(np.float32)
    assert np.all(scale >= np.float32(2.0 ** -126))
    q_div = np.rint(rows / scale[:, None])
    r0 = (np.float32(1.0) / scale).astype(np.float32)
    misrounded = 0
    for r in (np.nextafter(r0, np.float32(0)), r0, np.nextafter(r0, np.float32(np.inf))):
        y = rows.astype(np.float64) * r.astype(np.float64)[:, None]  # exact products
        n = np.rint(y)                                                 # ties to even
        ef = (y - n).astype(np.float32)                                # one rounding
        band = np.abs(ef) >= np.float32(0.5 - 2.0 ** -14)
        wrong = n != q_div
        assert not np.any(wrong & ~band)
        misrounded += int(wrong.sum())
    assert misrounded > 1000   # the rows do reach the ties a plain reciprocal gets wrong


def _rn32_of_sum(s, err):
    # fp32 round-to-nearest-even of s + err, s float64 and |err| below half an ulp of s
    # (the error term of an error-free sum): s rounds alone unless it sits exactly on an
    # fp32 midpoint, where the sign of err decides.
    import numpy as np
    a = s.astype(np.float32)
    lo = np.nextafter(a, np.float32(-np.inf))
    hi = np.nextafter(a, np.float32(np.inf))
    mid_lo = (a.astype(np.float64) + lo.astype(np.float64)) / 2
    mid_hi = (a.astype(np.float64) + hi.astype(np.float64)) / 2
    out = a.copy()
    down = (s == mid_lo) & (err < 0)
    up = (s == mid_hi) & (err > 0)
    out[down] = lo[down]
    out[up] = hi[up]
    return out


def _div127_corrected(x):
    # The kernels' scale for amax in [2^-90, 2^127): q = RN(x RN(1/127)), rem = fma(-q,
    # 127, x), scale = fma(rem, RN(1/127), q), every operation rounded once to fp32
    # (nearest, ties to even), emulated exactly in float64.
    import numpy as np
    r = np.float32(1.0) / np.float32(127.0)
    q = (x * r).astype(np.float32)
    rem_exact = x.astype(np.float64) - 127.0 * q.astype(np.float64)  # exact in float64
    rem = rem_exact.astype(np.float32)
    assert np.array_equal(rem.astype(np.float64), rem_exact)         # the fma is exact
    p = rem.astype(np.float64) * np.float64(r)                        # exact (24 x 24 bits)
    s = q.astype(np.float64) + p
    bb = s - q.astype(np.float64)
    err = (q.astype(np.float64) - (s - bb)) + (p - bb)                # two-sum error
    return _rn32_of_sum(s, err)


def test_scale_division_by_127_corrected_product():
    # The per-row scale amax / 127 must be the IEEE fp32 quotient. The kernels form it as a
    # product with RN(1/127) corrected by one fma on the exact remainder. The rounding of
    # that correction depends on the significand alone inside the range (no subnormal
    # intermediate, no overflow), so every significand of one binade is checked against
    # numpy's IEEE division, plus random values over the whole range; the uncorrected
    # product is wrong for a few percent of them, which the check must see.
    import numpy as np
    rng = np.random.default_rng(127)
    for part in range(4):
        bits = np.uint32(127 << 23) + np.arange(part << 21, (part + 1) << 21, dtype=np.uint32)
        x = bits.view(np.float32)
        ref = x / np.float32(127.0)
        got = _div127_corrected(x)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        plain = (x * (np.float32(1.0) / np.float32(127.0))).astype(np.float32)
        assert np.count_nonzero(plain != ref) > 50000
    e = rng.integers(-90, 127, 1 << 20)
    x = np.ldexp(1.0 + rng.random(1 << 20), e).astype(np.float32)
    x = x[np.isfinite(x) & (x < np.float32(2.0 ** 127))]
    got = _div127_corrected(x)
    assert np.array_equal(got.view(np.uint32), (x / np.float32(127.0)).view(np.uint32))
