"""attn_decode_int8p (decode / verify with int8 softmax weights on the int8 matrix cores)
against the oracle: max abs error <= 1e-2 * max|V_deq| vs exact attention and <= 1e-3 *
max|V_deq| vs the int8-P rule (a diagnostic of the code path), for every partition size;
results do not depend on the partition beyond rounding. ("INT8 KV and INT8 MMAC
attention on a gfx936 DCU" §3.3: INT8 PV decode, 256-token partitions; vLLM docs page,
"The selection law".)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import DecodeSetup, need_gpu, say

pytestmark = pytest.mark.gpu

TOL_A = 1e-2
TOL_B = 1e-3


def _check(st, out, seqs=None):
    seqs = sorted(st.ref) if seqs is None else seqs
    wa = wb = 0.0
    for s in seqs:
        ea = float(np.max(np.abs(out[s] - st.oracle_verify(s))))
        eb = float(np.max(np.abs(out[s] - st.oracle_int8p(s))))
        wa, wb = max(wa, ea), max(wb, eb)
        assert ea <= TOL_A * st.vmax, (s, int(st.case.context_lens[s]), ea, st.vmax)
        assert eb <= TOL_B * st.vmax, (s, int(st.case.context_lens[s]), eb, st.vmax)
    say(f"  worst err vs exact {wa:.3e} (bound {TOL_A * st.vmax:.3e}), vs int8-P rule {wb:.3e} "
        f"(bound {TOL_B * st.vmax:.3e})")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_int8p_decode_configs(cfg):
    need_gpu()
    case = workloads.config_case(cfg)
    rows = lib.attn_decode_partition_rows(case.num_seqs, case.max_context_len, 4)
    say(f"attn_decode_int8p config {cfg} (partition {rows})")
    st = DecodeSetup(case)
    _check(st, st.run_int8p())


@pytest.mark.parametrize("part", [64, 128, 256, 512])
def test_int8p_every_partition_size_agrees(part):
    need_gpu()
    ctx = [1, 15, 64, 65, 300, 511, 513, 1100, 2049]
    case = workloads.make_decode_case(90, ctx, pages="random", k_outliers=4, extra_pages=3)
    st = DecodeSetup(case)
    out = st.run_int8p(partition_rows=part)
    say(f"attn_decode_int8p partition {part}, contexts {ctx}")
    _check(st, out)
    ref = st.run_int8p(partition_rows=512)
    d = float(np.max(np.abs(out - ref)))
    say(f"  |partition {part} - partition 512| = {d:.3e}")
    assert d <= 1e-5 * st.vmax


@pytest.mark.parametrize("nq", [2, 4, 8])
def test_int8p_verify_rows(nq):
    need_gpu()
    ctx = [nq, 70, 512 + nq - 2, 1030]
    case = workloads.make_decode_case(91 + nq, ctx, pages="random", k_outliers=4,
                                      q_rows_per_seq=nq)
    say(f"attn_decode_int8p nq={nq}, contexts {ctx}")
    st = DecodeSetup(case)
    _check(st, st.run_int8p())
    _check(st, st.run_int8p(partition_rows=64))


@pytest.mark.parametrize("n_kv,nq", [(1, 1), (3, 4), (8, 2)])
def test_int8p_other_kv_head_counts(n_kv, nq):
    # grid, tiles and merge at other group counts (6 query heads per KV head); the law picks
    # the partition from the head count
    need_gpu()
    ctx = [nq, 40, 600, 1500]
    case = workloads.make_decode_case(310 + n_kv, ctx, pages="random", k_outliers=4, extra_pages=2,
                                      q_rows_per_seq=nq, n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    rows = lib.attn_decode_partition_rows(len(ctx), max(ctx), n_kv)
    say(f"attn_decode_int8p nq={nq} contexts {ctx} with {n_kv} KV heads (partition {rows})")
    st = DecodeSetup(case)
    _check(st, st.run_int8p())


def test_int8p_batch_flattened_grid():
    # 20 sequences with 512-key partitions: the flattened grid of real work items; the
    # same batch at 64-key partitions keeps the grid (both to the oracle), and rows before
    # their context (context 2 with 4 rows) are 0
    need_gpu()
    nq = 4
    ctx = [2, 70, 512 + nq - 2, 1030, 3000] * 4
    case = workloads.make_decode_case(97, ctx, pages="random", k_outliers=4, q_rows_per_seq=nq)
    say(f"attn_decode_int8p nq={nq}, {len(ctx)} sequences")
    st = DecodeSetup(case)
    out = st.run_int8p(partition_rows=512)
    assert np.all(out[0, :2] == 0.0)
    _check(st, out)
    _check(st, st.run_int8p(partition_rows=64))


def test_int8p_batch_flattened_grid_single_partition():
    # 18 sequences, every context within one 512-key partition: the flattened grid writes
    # the normalized rows itself (no merge stage)
    need_gpu()
    nq = 2
    ctx = [1, 2, 37, 300, 511, 512] * 3
    case = workloads.make_decode_case(98, ctx, pages="random", k_outliers=4, q_rows_per_seq=nq)
    say(f"attn_decode_int8p nq={nq}, {len(ctx)} sequences of at most 512 keys")
    st = DecodeSetup(case)
    out = st.run_int8p(partition_rows=512)
    assert np.all(out[0, :1] == 0.0)
    _check(st, out)


def test_int8p_rows_before_the_context_are_zero():
    need_gpu()
    case = workloads.make_decode_case(95, [2, 3], pages="random", q_rows_per_seq=4)
    st = DecodeSetup(case)
    out = st.run_int8p(partition_rows=64)
    say("attn_decode_int8p nq=4 with contexts 2 and 3")
    assert np.all(out[0, :2] == 0.0) and np.all(out[1, :1] == 0.0)
    _check(st, out)


def test_int8p_workspace_checks():
    need_gpu()
    case = workloads.make_decode_case(96, [3000], pages="random")
    st = DecodeSetup(case)
    need = lib.attn_decode_int8p_workspace_bytes(1, 1, 3000, 24, 4, partition_rows=64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.Int8AttnError):
        lib.attn_decode_int8p(st.q_all, st.cache, st.table, st.ctx, 3000, partition_rows=64,
                              workspace=ws[:need - 256])
    with pytest.raises(lib.Int8AttnError):
        lib.attn_decode_int8p(st.q_all, st.cache, st.table, st.ctx, 3000, partition_rows=96,
                              workspace=ws)
    out = lib.attn_decode_int8p(st.q_all, st.cache, st.table, st.ctx, 3000, partition_rows=64,
                                workspace=ws)
    torch.cuda.synchronize()
    _check(st, out.cpu().numpy())
