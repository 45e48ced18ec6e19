"""attn_prefill_chunk_split (short causal chunks: keys cut into partitions of whole
64-key blocks, one workgroup per partition, log-sum-exp merge; chunks of at most 8 rows on
the int8-P decode kernel) against the oracle, to the bounds of the one-pass chunk: max abs error <= 1e-2 * max|V_deq| vs exact attention and
<= 1e-3 * max|V_deq| vs the int8-P emulation (the weight codes stay per aligned 64-key
block, so the emulation is the same). Chunks that the route leaves to the one pass must
equal attn_prefill_chunk bit for bit.
("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.2, §3.3: partitions and their
merge as in the decode, the int8 weight rule inside each.)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import PrefillSetup, need_gpu, say

pytestmark = pytest.mark.gpu

TOL_A = 1e-2
TOL_B = 1e-3


def _split(st, causal=True, q_scales=None, q=None):
    c = st.case
    out = lib.attn_prefill_chunk_split(st.q if q is None else q, st.cache, st.table,
                                       c.context_len, causal, q_scales=q_scales)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(st, rows, out):
    ref_a = st.oracle(rows)
    ref_b = st.oracle(rows, int8p=True)
    ea = float(np.max(np.abs(out[rows] - ref_a)))
    eb = float(np.max(np.abs(out[rows] - ref_b)))
    say(f"  rows {len(rows)}: err vs exact {ea:.3e} (bound {TOL_A * st.vmax:.3e}), "
        f"vs int8-P emulation {eb:.3e} (bound {TOL_B * st.vmax:.3e})")
    assert ea <= TOL_A * st.vmax
    assert eb <= TOL_B * st.vmax


@pytest.mark.parametrize("ctx,n_new,n_kv", [
    (3000, 1, 4),      # at most 8 rows: the int8-P decode kernel
    (3000, 5, 4),
    (20000, 3, 1),
    (5, 5, 4),         # ... with a single key partition (no merge)
    (3000, 40, 4),     # two query blocks, ragged second
    (3000, 100, 4),    # four query blocks: rows end in different partitions
    (20000, 12, 1),    # one KV head: 157 partitions per row
    (1000, 500, 4),    # early query blocks stop before the last partition; rows without
                       # a key in a partition keep an empty state there
    (2000, 70, 3),     # three KV heads
    (130, 33, 4),      # three 64-key blocks, ragged tail
])
def test_split_small(ctx, n_new, n_kv):
    need_gpu()
    need = lib.attn_prefill_chunk_split_workspace_bytes(n_new, ctx, True, 6 * n_kv, n_kv)
    say(f"attn_prefill_chunk_split ctx={ctx} n_new={n_new} n_kv={n_kv}: workspace {need} B")
    assert need > 0  # these chunks take the split route
    case = workloads.make_prefill_case(90 + ctx + n_new, ctx, n_new, k_outliers=4,
                                       extra_pages=2, n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    st = PrefillSetup(case)
    out = _split(st)
    _check(st, np.arange(n_new), out)
    one = st.run()
    d = float(np.max(np.abs(out - one)))
    say(f"  split vs one pass: {d:.3e}")
    assert d <= TOL_B * st.vmax


def test_split_long_context_sampled():
    # A 64-token chunk at the end of a 32768-token context: 8 one-pass workgroups,
    # 256 with the split.
    need_gpu()
    ctx, n_new = 32768, 64
    say(f"attn_prefill_chunk_split ctx={ctx} n_new={n_new}")
    st = PrefillSetup(workloads.make_prefill_case(7, ctx, n_new, k_outliers=4))
    out = _split(st)
    _check(st, np.array([0, 1, 15, 16, 31, 32, 47, 62, 63]), out)


def test_long_context_both_routes_sampled():
    # the longest context of the decode workloads (131,072 keys): a 256-row chunk on the
    # split route (8 query blocks x 4 heads -> 8 partitions of 256 blocks) and on the one
    # pass, sampled rows against the oracle
    need_gpu()
    ctx, n_new = 131072, 256
    say(f"attn_prefill_chunk(_split) ctx={ctx} n_new={n_new}")
    st = PrefillSetup(workloads.make_prefill_case(17, ctx, n_new, k_outliers=4))
    rows = np.array([0, 31, 32, 100, 200, 255])
    split = _split(st)
    _check(st, rows, split)
    one = st.run()
    _check(st, rows, one)
    assert np.max(np.abs(split - one)) <= TOL_B * st.vmax


@pytest.mark.parametrize("ctx,n_new,causal", [
    (1500, 200, False),   # non-causal: always the one pass
    (5000, 1100, True),   # 35 query blocks x 4 KV heads = 140 workgroups: the one pass
    (100, 20, True),      # two 64-key blocks, one query block: split into two
    (64, 10, True),       # one 64-key block: the one pass
])
def test_split_route_boundaries(ctx, n_new, causal):
    need_gpu()
    need = lib.attn_prefill_chunk_split_workspace_bytes(n_new, ctx, causal, 24, 4)
    say(f"attn_prefill_chunk_split ctx={ctx} n_new={n_new} causal={causal}: workspace {need} B")
    st = PrefillSetup(workloads.make_prefill_case(30 + n_new, ctx, n_new, k_outliers=4))
    out = _split(st, causal)
    one = st.run(causal)
    if need == 0:
        assert np.array_equal(out, one)
    else:
        assert np.max(np.abs(out - one)) <= TOL_B * st.vmax
        _check(st, np.arange(n_new), out)


def test_split_q8_matches_bf16_form():
    need_gpu()
    say("attn_prefill_chunk_split_q8 with q_quant codes vs the bf16 form")
    st = PrefillSetup(workloads.make_prefill_case(11, 2500, 50, k_outliers=4))
    codes, scales = lib.q_quant(st.q)
    a = _split(st)
    b = _split(st, q=codes, q_scales=scales)
    assert np.array_equal(a, b)


def test_split_workspace_reuse_and_smaller_chunk():
    # One workspace for two calls in a row (the second with fewer rows and partitions):
    # leftovers of the first never reach the second's result.
    need_gpu()
    say("attn_prefill_chunk_split: a shared workspace over two calls")
    st1 = PrefillSetup(workloads.make_prefill_case(12, 6000, 90, k_outliers=4))
    st2 = PrefillSetup(workloads.make_prefill_case(13, 700, 7, k_outliers=4))
    n1 = lib.attn_prefill_chunk_split_workspace_bytes(90, 6000, True, 24, 4)
    ws = torch.full((n1,), 0xff, dtype=torch.uint8, device="cuda")  # NaN bit patterns
    a = lib.attn_prefill_chunk_split(st1.q, st1.cache, st1.table, 6000, True, workspace=ws)
    b = lib.attn_prefill_chunk_split(st2.q, st2.cache, st2.table, 700, True, workspace=ws)
    torch.cuda.synchronize()
    _check(st1, np.arange(90), a.cpu().numpy())
    _check(st2, np.arange(7), b.cpu().numpy())
