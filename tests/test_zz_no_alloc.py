"""attn_decode_noalloc (partials in the library's fixed per-GPU array, no workspace)
against attn_decode (caller workspace) on the same inputs, through the C-ABI: two calls in
a row, the second on a smaller batch, each bit-identical to attn_decode and within the
fp32-class bar of the oracle. ("dot4-flash-attention" README route table: split-K decode
+ merge; "INT8 KV and INT8 MMAC attention on a gfx936 DCU" §3.3.)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import DecodeSetup, need_gpu, say

pytestmark = pytest.mark.gpu

TOL = 1e-4


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    need_gpu()
    big = DecodeSetup(workloads.make_decode_case(501, [32768, 5000, 700, 1], pages="random",
                                                 k_outliers=4))
    small = DecodeSetup(workloads.make_decode_case(502, [1300, 17], pages="random"))
    for name, st in (("4 sequences up to 32,768 keys", big), ("2 sequences up to 1,300 keys", small)):
        c = st.case
        say(f"attn_decode_noalloc vs attn_decode: {name}")
        out_na = torch.full((c.num_seqs, c.n_q_heads, c.head_dim), float("nan"), device="cuda")
        lib.attn_decode_noalloc(st.q, st.cache, st.table, st.ctx, c.max_context_len, out=out_na)
        ref = lib.attn_decode(st.q, st.cache, st.table, st.ctx, c.max_context_len)
        torch.cuda.synchronize()
        a, b = out_na.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(a, b)
        worst = max(float(np.max(np.abs(a[s] - st.oracle_out(s)))) for s in range(c.num_seqs))
        say(f"  bit-identical to attn_decode; worst err vs oracle {worst:.3e} "
            f"(bound {TOL * st.vmax:.3e})")
        assert worst <= TOL * st.vmax


def test_noalloc_refuses_a_batch_beyond_its_array():
    need_gpu()
    st = DecodeSetup(workloads.make_decode_case(503, [600], pages="random"))
    out = torch.full((1, 24, 256), 7.0, device="cuda")
    with pytest.raises(lib.Int8AttnError) as e:
        lib.attn_decode_noalloc(st.q, st.cache, st.table, st.ctx, 2 ** 22, out=out)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
