"""The measurement kernels read what they claim: every 16-byte chunk of the streaming
read's buffer, and every K/V page and scale that the page-gather read's block table names,
exactly once (the XOR of all sink words equals the XOR of the words read; a chunk skipped,
or read twice, changes it). Both are timed by bench.py as ceilings for the decode."""
import numpy as np
import pytest
import torch

import int8_kv_cache_amd as lib
from tests.gpu_support import need_gpu, say

pytestmark = pytest.mark.gpu


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(), initial=0))


@pytest.mark.parametrize("nbytes,wg", [(16 * 1000, 7), (1 << 20, 256), ((1 << 20) + 48, 64)])
def test_stream_read_reads_every_chunk_once(nbytes, wg):
    need_gpu()
    say(f"ceiling_stream_read {nbytes} B, {wg} workgroups")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    sink = torch.zeros(4 * wg, dtype=torch.int32, device="cuda")
    lib.ceiling_stream_read(src, wg, sink)
    torch.cuda.synchronize()
    assert _xor_words(sink.cpu().numpy()) == _xor_words(host)


@pytest.mark.parametrize("n_blocks,ppw", [(50, 8), (64, 16), (37, 32), (1, 8)])
def test_page_gather_reads_every_named_page_once(n_blocks, ppw):
    need_gpu()
    say(f"ceiling_page_gather {n_blocks} pages, {ppw} per workgroup")
    num_pages, H = 96, 4
    rng = np.random.default_rng(1000 + n_blocks)
    cache = lib.alloc_cache(num_pages, H, "cuda")
    kc = rng.integers(-127, 128, cache.k_cache.numel(), dtype=np.int8)
    vc = rng.integers(-127, 128, cache.v_cache.numel(), dtype=np.int8)
    ks = rng.random(cache.k_scale.numel(), dtype=np.float32)
    vs = rng.random(cache.v_scale.numel(), dtype=np.float32)
    for t, a in ((cache.k_cache, kc), (cache.v_cache, vc), (cache.k_scale, ks), (cache.v_scale, vs)):
        t.copy_(torch.from_numpy(a))
    table = rng.permutation(num_pages)[:n_blocks].astype(np.int32)
    if n_blocks > 3:
        table[3] = num_pages + 5          # outside the pool: page 0 is read instead
    expect = 0
    for pr in table:
        p = int(pr) if 0 <= pr < num_pages else 0
        for g in range(H):
            blk = (p * H + g)
            expect ^= _xor_words(kc[blk * 4096:(blk + 1) * 4096]) ^ _xor_words(vc[blk * 4096:(blk + 1) * 4096])
            expect ^= _xor_words(ks[blk * 16:(blk + 1) * 16]) ^ _xor_words(vs[blk * 16:(blk + 1) * 16])
    nx = -(-n_blocks // ppw)
    sink = torch.zeros(4 * nx * H, dtype=torch.int32, device="cuda")
    nbytes = lib.ceiling_page_gather(cache, torch.from_numpy(table).cuda(), n_blocks, ppw, sink)
    torch.cuda.synchronize()
    assert nbytes == n_blocks * (H * (2 * 4096 + 2 * 64) + 4)
    assert _xor_words(sink.cpu().numpy()) == expect
