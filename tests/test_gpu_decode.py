"""attn_decode (split-K over 512-row partitions + log-sum-exp merge) against the exact
FP64 oracle: max abs error <= 1e-4 * max|V_deq| (P and V kept at fp32 precision).
("dot4-flash-attention" README route table split-K; "INT8 KV and INT8 MMAC attention on
a gfx936 DCU" §3.3.)"""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
import workloads
from tests.gpu_support import DecodeSetup, need_gpu, say, up

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _check_all(setup, seqs=None):
    out = setup.run()
    seqs = sorted(setup.ref) if seqs is None else seqs
    worst = 0.0
    for s in seqs:
        ref = setup.oracle_out(s)
        err = float(np.max(np.abs(out[s] - ref)))
        worst = max(worst, err)
        assert err <= TOL * setup.vmax, (s, int(setup.case.context_lens[s]), err, setup.vmax)
    say(f"  worst abs err {worst:.3e}  (bound {TOL * setup.vmax:.3e})")
    return out


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_decode_configs(cfg):
    need_gpu()
    say(f"attn_decode config {cfg}")
    _check_all(DecodeSetup(workloads.config_case(cfg)))


EDGE_CTX = [1, 2, 15, 16, 17, 63, 64, 65, 100, 511, 512, 513, 1023, 1024, 1300, 2049]


@pytest.mark.parametrize("n_seqs", [15, 16, 40])
def test_decode_edge_contexts_batched(n_seqs):
    # 15 sequences: the (partition, head, sequence) grid; 16 and more: the flattened grid
    # of real work items
    need_gpu()
    ctx = (EDGE_CTX * 3)[:n_seqs]
    say(f"attn_decode edge contexts, {n_seqs} sequences: {ctx}")
    case = workloads.make_decode_case(41, ctx, pages="random", k_outliers=4, extra_pages=5)
    _check_all(DecodeSetup(case))


@pytest.mark.parametrize("n_seqs", [3, 20])
def test_decode_zero_contexts_give_zeros(n_seqs):
    # a context length of 0 (or below 0) in the batch gives zeros for that sequence and
    # leaves the others exact, on both grids; all contexts <= 512 (no merge stage) and
    # longer ones
    need_gpu()
    rng = np.random.default_rng(n_seqs)
    for hi in (512, 3000):
        ctx = list(rng.integers(1, hi + 1, n_seqs))
        say(f"attn_decode {n_seqs} sequences, contexts up to {hi}, two set to 0 and -5")
        st = DecodeSetup(workloads.make_decode_case(48 + hi, ctx, pages="random", k_outliers=4))
        zero = [0, n_seqs - 1]
        c = st.case.context_lens.copy()
        c[zero[0]], c[zero[1]] = 0, -5
        st.ctx = up(c)
        out = st.run()
        for s in zero:
            assert np.all(out[s] == 0.0)
        for s in range(1, n_seqs - 1):
            assert np.max(np.abs(out[s] - st.oracle_out(s))) <= TOL * st.vmax


def test_decode_flat_grid_one_kv_head():
    need_gpu()
    ctx = [700, 1, 5000, 513, 64, 2100, 90, 1024] * 3
    say(f"attn_decode {len(ctx)} sequences with 1 KV head x 6 query heads")
    case = workloads.make_decode_case(85, ctx, pages="random", k_outliers=4, n_q_heads=6,
                                      n_kv_heads=1)
    _check_all(DecodeSetup(case))


def test_ctx1_returns_v_exactly():
    need_gpu()
    case = workloads.make_decode_case(42, [1, 1, 1], pages="random")
    st = DecodeSetup(case)
    out = st.run()
    for s in range(3):
        kc, ks, vc, vs = st.ref[s]
        exp = (vc[0].astype(np.float32) * vs[0][:, None]).astype(np.float32)   # fl32(code*scale)
        got = out[s].reshape(4, 6, 256)
        for g in range(4):
            assert np.array_equal(got[g], np.broadcast_to(exp[g], (6, 256)))


def test_identity_vs_permuted_pages_agree():
    need_gpu()
    a = DecodeSetup(workloads.make_decode_case(43, [700], pages="identity"))
    b = DecodeSetup(workloads.make_decode_case(43, [700], pages="random"))
    assert not np.array_equal(a.case.block_table, b.case.block_table)
    assert np.array_equal(a.run(), b.run())


def test_distinct_v_bytes_detect_half_reads():
    # Every (token, dim) of V gets its own value so that a load reading half a vector,
    # the wrong page or the wrong token group cannot go unnoticed (gfx936 article §5.4).
    need_gpu()
    case = workloads.make_decode_case(44, [1000], pages="random")
    st = DecodeSetup(case, keep=[0])
    k, v, q = case.seq_data(0)
    t = np.arange(1000)[:, None, None]; d = np.arange(256)[None, None, :]; h = np.arange(4)[None, :, None]
    v2 = (((t * 7 + d * 13 + h * 5) % 251) - 125).astype(np.float32)
    v2[:, :, 0] = 127.0                                  # scale exactly 1: codes = values
    lib.kv_quant_write(up(k), up(v2), up(case.seq_slots(0)), st.cache)
    from oracle import quant
    vc, vs = quant.quantize_rows(v2)
    st.ref[0] = st.ref[0][:2] + (vc, vs)
    st.vmax = 127.0
    _check_all(st)


def test_workspace_reuse_smaller_call_and_stream():
    need_gpu()
    big = DecodeSetup(workloads.make_decode_case(45, [5000, 3000], pages="random"))
    ws = torch.empty(lib.attn_decode_workspace_bytes(2, 5000, 24), dtype=torch.uint8, device="cuda")
    small = DecodeSetup(workloads.make_decode_case(46, [900, 20], pages="random"))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1 = lib.attn_decode(big.q, big.cache, big.table, big.ctx, 5000, workspace=ws)
        o2 = lib.attn_decode(small.q, small.cache, small.table, small.ctx, 900, workspace=ws)
    torch.cuda.synchronize()
    for st, o in ((big, o1), (small, o2)):
        for sq in range(2):
            assert np.max(np.abs(o.cpu().numpy()[sq] - st.oracle_out(sq))) <= TOL * st.vmax


def test_workspace_too_small_is_rejected():
    need_gpu()
    st = DecodeSetup(workloads.make_decode_case(47, [600], pages="random"))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.full((1, 24, 256), 7.0, device="cuda")
    with pytest.raises(lib.Int8AttnError) as e:
        lib.attn_decode(st.q, st.cache, st.table, st.ctx, 600, out=out, workspace=ws)
    assert e.value.code == -3
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("n_kv", [1, 3, 8])
def test_decode_other_kv_head_counts(n_kv):
    need_gpu()
    ctx = [1, 700, 1537]
    say(f"attn_decode ctx {ctx} with {n_kv} KV heads x 6 query heads")
    case = workloads.make_decode_case(80 + n_kv, ctx, pages="random", k_outliers=4,
                                      n_q_heads=6 * n_kv, n_kv_heads=n_kv)
    _check_all(DecodeSetup(case))
