"""Large decode / verify batches with short ragged contexts, some of them 0, against the
oracle: batches of 200, 1,024 and 4,096 sequences run the flattened grid of real work
items whose prefix scan gives each lane several sequences and whose sequence lookup takes
its second ballot step (more than 64 sequences). Every sequence is compared.
("dot4-flash-attention" README route table: split-K decode; "INT8 KV and INT8 MMAC
attention on a gfx936 DCU" §3.3: decode over paged INT8 K/V with a block table.)"""
import numpy as np
import pytest

import workloads
from tests.gpu_support import DecodeSetup, need_gpu, say, up

pytestmark = pytest.mark.gpu

TOL = 1e-4      # fp32-class weights
TOL_A = 1e-2    # int8 weights vs exact attention
TOL_B = 1e-3    # int8 weights vs the int8-P rule


def _batch(seed, n_seqs, nq=1, hi=1100):
    rng = np.random.default_rng([seed, n_seqs])
    ctx = rng.integers(1, hi + 1, n_seqs)
    ctx[rng.choice(n_seqs, 3, replace=False)] = rng.choice([1, 2, 16, 17, 512, 513], 3)
    case = workloads.make_decode_case(seed + n_seqs, list(ctx), pages="random", k_outliers=4,
                                      extra_pages=7, q_rows_per_seq=nq)
    st = DecodeSetup(case, threads=16)
    # a few padded batch slots: context 0 (and one negative) give zero rows
    zero = rng.choice(n_seqs, 4, replace=False)
    c = case.context_lens.copy()
    c[zero[:3]] = 0
    c[zero[3]] = -3
    st.ctx = up(c)
    return st, set(int(z) for z in zero)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_seqs", [200, 1024, 4096])
def test_decode_large_batches(n_seqs):
    need_gpu()
    st, zero = _batch(300, n_seqs)
    say(f"attn_decode {n_seqs} sequences, contexts 0..1100 ({sorted(zero)} set to 0 / -3)")
    out = st.run()
    worst = 0.0
    for s in range(n_seqs):
        if s in zero:
            assert np.all(out[s] == 0.0), s
            continue
        err = float(np.max(np.abs(out[s] - st.oracle_out(s))))
        worst = max(worst, err)
        assert err <= TOL * st.vmax, (s, int(st.case.context_lens[s]), err)
    say(f"  worst abs err {worst:.3e} (bound {TOL * st.vmax:.3e})")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_seqs,nq", [(200, 2), (1024, 4)])
def test_verify_and_int8p_large_batches(n_seqs, nq):
    need_gpu()
    st, zero = _batch(400, n_seqs, nq=nq)
    say(f"attn_verify / attn_decode_int8p nq={nq}, {n_seqs} sequences, contexts 0..1100")
    ver = st.run_verify()
    i8p = st.run_int8p()
    wv = wa = wb = 0.0
    for s in range(n_seqs):
        if s in zero:
            assert np.all(ver[s] == 0.0) and np.all(i8p[s] == 0.0), s
            continue
        ev = float(np.max(np.abs(ver[s] - st.oracle_verify(s))))
        ea = float(np.max(np.abs(i8p[s] - st.oracle_verify(s))))
        eb = float(np.max(np.abs(i8p[s] - st.oracle_int8p(s))))
        wv, wa, wb = max(wv, ev), max(wa, ea), max(wb, eb)
        assert ev <= TOL * st.vmax, (s, ev)
        assert ea <= TOL_A * st.vmax and eb <= TOL_B * st.vmax, (s, ea, eb)
    say(f"  verify worst {wv:.3e} (bound {TOL * st.vmax:.3e}); int8-P worst vs exact {wa:.3e}, "
        f"vs rule {wb:.3e}")
