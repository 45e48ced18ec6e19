"""attn_prefill_chunk (one online-softmax pass, int8 P per 64-key block on int8 MFMA)
against the oracle: max abs error <= 1e-2 * max|V_deq| vs exact attention, and <= 1e-3 *
max|V_deq| vs the int8-P emulation (a diagnostic of the P quantization).
("INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.2, §3.3; "#3381 prompt QSA attention
without the decode kernel's split and merge", Validation: checked against an FP64 host
reference and against the decode kernel.)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import PrefillSetup, need_gpu, say, up

pytestmark = pytest.mark.gpu

TOL_A = 1e-2
TOL_B = 1e-3


def _check(st, rows, causal=True):
    out = st.run(causal)
    ref_a = st.oracle(rows, causal)
    ref_b = st.oracle(rows, causal, int8p=True)
    ea = float(np.max(np.abs(out[rows] - ref_a)))
    eb = float(np.max(np.abs(out[rows] - ref_b)))
    say(f"  rows {len(rows)}: err vs exact {ea:.3e} (bound {TOL_A * st.vmax:.3e}), "
        f"vs int8-P emulation {eb:.3e} (bound {TOL_B * st.vmax:.3e})")
    assert ea <= TOL_A * st.vmax
    assert eb <= TOL_B * st.vmax
    return out


@pytest.mark.parametrize("ctx,n_new,causal", [
    (300, 300, True),      # no history, ragged last page and block
    (1000, 77, True),      # history + ragged chunk
    (1, 1, True),          # single key
    (64, 16, True),        # exact tiles
    (1500, 200, False),    # non-causal
    (130, 33, True),
])
def test_prefill_small(ctx, n_new, causal):
    need_gpu()
    say(f"attn_prefill_chunk ctx={ctx} n_new={n_new} causal={causal}")
    st = PrefillSetup(workloads.make_prefill_case(50 + ctx, ctx, n_new, k_outliers=4, extra_pages=3))
    _check(st, np.arange(n_new), causal)


def test_prefill_rows_match_decode_at_matching_context():
    need_gpu()
    case = workloads.make_prefill_case(60, 2500, 130, k_outliers=4)
    st = PrefillSetup(case)
    out = st.run()
    rows = [0, 1, 64, 129]
    pos0 = case.context_len - case.n_new
    S = len(rows)
    ctx = np.array([pos0 + t + 1 for t in rows], np.int32)
    table = np.tile(case.block_table, (S, 1))
    q = st.q[torch.as_tensor(rows, device="cuda")]
    dec = lib.attn_decode(q.contiguous(), st.cache, up(table), up(ctx), int(ctx.max()))
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    for i, t in enumerate(rows):
        assert np.max(np.abs(out[t] - dec[i])) <= TOL_A * st.vmax


@pytest.mark.parametrize("n_kv", [1, 2, 3, 5])
def test_prefill_other_kv_head_counts(n_kv):
    # 1 and 2 KV heads take the per-XCD tile order (with padding workgroups when the chunk
    # has fewer query blocks than XCDs per head); 3 and 5 take the plain order.
    need_gpu()
    say(f"attn_prefill_chunk ctx=400 n_new=90 with {n_kv} KV heads x 6 query heads")
    case = workloads.make_prefill_case(70 + n_kv, 400, 90, k_outliers=4,
                                       n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    st = PrefillSetup(case)
    _check(st, np.arange(case.n_new))
