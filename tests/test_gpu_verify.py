"""attn_verify (nq query rows per sequence on the split-K kernel + log-sum-exp merge)
against the exact FP64 oracle: max abs error <= 1e-4 * max|V_deq|, the one-row bar
(P and V kept at fp32 precision). ("dot4-flash-attention" README: MTP verify runs a
few query rows and split-K decode is to be extended to them; vLLM docs page, "Row shape
routing": verify rows on a multi-row kernel, one row on the one-row kernel.)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import DecodeSetup, need_gpu, say

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _check(st, out, seqs=None):
    seqs = sorted(st.ref) if seqs is None else seqs
    worst = 0.0
    for s in seqs:
        ref = st.oracle_verify(s)
        err = float(np.max(np.abs(out[s] - ref)))
        worst = max(worst, err)
        assert err <= TOL * st.vmax, (s, int(st.case.context_lens[s]), err, st.vmax)
    say(f"  worst abs err {worst:.3e}  (bound {TOL * st.vmax:.3e})")


@pytest.mark.parametrize("nq", [2, 3, 4, 8])
def test_verify_ragged_contexts(nq):
    need_gpu()
    # rows straddle page edges (16), partition edges (512, 1024) and the wave edge (64)
    ctx = [nq, 17, 64 + nq - 1, 300, 512 + nq - 2, 513, 1024 + 3, 2049]
    say(f"attn_verify nq={nq} contexts {ctx}")
    case = workloads.make_decode_case(70 + nq, ctx, pages="random", k_outliers=4, extra_pages=3,
                                      q_rows_per_seq=nq)
    st = DecodeSetup(case)
    _check(st, st.run_verify())


@pytest.mark.parametrize("n_kv,nq", [(1, 4), (3, 2), (8, 3)])
def test_verify_other_kv_head_counts(n_kv, nq):
    # the (partition, KV head, sequence) grid, the query-row tiles of a group and the merge's
    # head index at other group counts (6 query heads per KV head)
    need_gpu()
    ctx = [nq, 40, 600, 1500]
    say(f"attn_verify nq={nq} contexts {ctx} with {n_kv} KV heads x 6 query heads")
    case = workloads.make_decode_case(300 + n_kv, ctx, pages="random", k_outliers=4, extra_pages=2,
                                      q_rows_per_seq=nq, n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    st = DecodeSetup(case)
    _check(st, st.run_verify())


@pytest.mark.parametrize("nq", [2, 4])
def test_verify_batch_flattened_grid(nq):
    # 24 sequences: the flattened grid of real work items (batches of 16 and more)
    need_gpu()
    ctx = [nq, 17, 64 + nq - 1, 300, 512 + nq - 2, 513, 1024 + 3, 2049] * 3
    say(f"attn_verify nq={nq}, {len(ctx)} sequences")
    case = workloads.make_decode_case(90 + nq, ctx, pages="random", k_outliers=4, extra_pages=3,
                                      q_rows_per_seq=nq)
    st = DecodeSetup(case)
    _check(st, st.run_verify())


def test_verify_batch_flattened_grid_single_partition():
    # 18 sequences of at most 512 keys: the flattened grid without a merge stage
    need_gpu()
    nq = 3
    ctx = [3, 20, 64, 300, 511, 512] * 3
    say(f"attn_verify nq={nq}, {len(ctx)} sequences of at most 512 keys")
    case = workloads.make_decode_case(99, ctx, pages="random", k_outliers=4, q_rows_per_seq=nq)
    st = DecodeSetup(case)
    _check(st, st.run_verify())


def test_verify_one_row_is_decode():
    need_gpu()
    case = workloads.make_decode_case(80, [1, 700, 1537], pages="random", k_outliers=4)
    st = DecodeSetup(case)
    a = st.run_verify()[:, 0]
    b = st.run()
    say("attn_verify nq=1 vs attn_decode")
    assert np.array_equal(a, b)


def test_verify_rows_match_decode_at_their_contexts():
    """Row i of a verify call equals a one-row decode whose context ends at the row."""
    need_gpu()
    nq, ctx = 4, 1030
    case = workloads.make_decode_case(81, [ctx], pages="random", k_outliers=4, q_rows_per_seq=nq)
    st = DecodeSetup(case)
    out = st.run_verify()[0]
    q = st.q_all[0]                                   # [nq, Hq, D]
    for i in range(nq):
        c_i = torch.tensor([ctx - nq + i + 1], dtype=torch.int32, device="cuda")
        d = lib.attn_decode(q[i:i + 1].contiguous(), st.cache, st.table, c_i, ctx)
        torch.cuda.synchronize()
        err = float(np.max(np.abs(out[i] - d.cpu().numpy()[0])))
        say(f"  row {i}: |verify - decode at ctx {ctx - nq + i + 1}| = {err:.3e}")
        assert err <= TOL * st.vmax


def test_verify_rows_before_the_context_are_zero():
    need_gpu()
    nq = 4
    case = workloads.make_decode_case(82, [2, 3], pages="random", q_rows_per_seq=nq)
    st = DecodeSetup(case)
    out = st.run_verify()
    say("attn_verify nq=4 with contexts 2 and 3")
    assert np.all(out[0, :2] == 0.0) and np.all(out[1, :1] == 0.0)
    _check(st, out)


def test_verify_workspace_reuse_and_streams():
    need_gpu()
    big = workloads.make_decode_case(83, [3000, 40], pages="random", q_rows_per_seq=3)
    small = workloads.make_decode_case(84, [600], pages="random", q_rows_per_seq=2)
    sb, ss = DecodeSetup(big), DecodeSetup(small)
    ws = torch.empty(lib.attn_verify_workspace_bytes(2, 3, 3000, 24), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    ob = sb.run_verify(workspace=ws)
    with torch.cuda.stream(side):
        os_ = lib.attn_verify(ss.q_all, ss.cache, ss.table, ss.ctx, 600, workspace=ws, stream=side)
    side.synchronize()
    say("attn_verify: one workspace, two shapes, two streams")
    _check(sb, ob)
    _check(ss, os_.cpu().numpy())
    with pytest.raises(lib.Int8AttnError):
        lib.attn_verify(sb.q_all, sb.cache, sb.table, sb.ctx, 3000, workspace=ws[:1024])


def test_verify_config3_context_sampled():
    """nq = 4 rows on one sequence of the 32k-context decode shape (random pages)."""
    need_gpu()
    case = workloads.make_decode_case(85, [32768], pages="random", q_rows_per_seq=4)
    say("attn_verify nq=4 at ctx 32768")
    st = DecodeSetup(case)
    _check(st, st.run_verify())
