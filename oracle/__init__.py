"""CPU reference ("oracle") for INT8-KV paged attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load
anything in this package: only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` use it. It shares no code with the HIP library
(`int8_kv_cache_amd/`) and imports nothing from it.

It is plain NumPy: fp32 semantics where the method fixes bit-exact results
(the quantizer), float64 everywhere else. Sources, cited by page title and section:

* "INT8 KV and INT8 MMAC attention on a gfx936 DCU" (gfx936 DCU上实现INT8 KV与INT8
  MMAC Attention推理优化, sourcefind forum): §2.1 quantization rule, §1.3 score and
  output formulas, §2.3 scale arrays, §3.3 decode partitions and merge.
* "dot4-flash-attention" (GitHub README): "Tile Inner Loop (pseudocode)" online
  softmax; the route table's split-K stage 1 + stage 2.
* "#3381 prompt QSA attention without the decode kernel's split and merge"
  (strata engine PR): "Approach" single online-softmax pass; "Validation" FP64
  host reference.

Modules:
  quant      -- per-row absmax/127 int8 quantizer, bf16 widening.
  paged      -- the paged cache byte layout (write and gather), by index formula.
  attention  -- exact softmax attention, split-K partials + log-sum-exp merge,
                int8-P emulation (per 64-key block), multi-row verify forms and a
                pure-Python brute force.
  rope       -- rotary embedding from a caller cos/sin table (fp32 pairwise rule) and
                the fused producer: rotate Q/K, quantize Q/K/V, paged K/V write.

Pins (tests/test_oracle_*.py) tie every function to something other than itself:
hand-derived tie cases, an fp64-then-round re-evaluation of the quantizer, the
2080 B/token byte accounting, brute force on tiny inputs, closed forms (ctx=1,
Q=0, equal keys, dominant key), softmax normalisation, merge = unsplit, page
permutation invariance, chunk row = decode at the matching context, verify rows =
decode at each row's context; RoPE against complex multiplication, exact quarter
turns, relative-position invariance of scores.
The int8-P emulation is pinned by brute force, an exact special case, its error
bound and a two-block case worked by hand from the rule; the pages print no worked
example of it.
"""
from . import quant, paged, attention, rope  # noqa: F401
