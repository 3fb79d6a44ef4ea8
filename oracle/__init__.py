"""CPU oracle for the DeepSeek Sparse Attention lightning indexer and its
top-k selector.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests, the smoke check of the graft entry point and the bench's
CPU-baseline leg may call it.  It shares no code with the HIP library; the
two meet only at the byte formats the seeded generators in ``synth`` write.

What it computes (plain definitions, fp64 throughout):

* ``formats``  -- decoding of the stored inputs: fp32, bf16 bit patterns and
  OCP FP8 E4M3FN codes times their fp32 scale.
* ``indexer``  -- the index score  I[t,s] = sum_i w[t,i] * ReLU(q[t,i].k[s] / sqrt(D))
  over the causal history s <= t (prefill) or over the cached context
  (paged decode), and the top-k selection by (score desc, index asc) with -1
  padding.  Vectorised with numpy.
* ``brute``    -- the same definitions as scalar pure-Python loops, used only
  on tiny inputs to pin ``indexer``.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: torch's own fp8/bf16 casts, closed-form codes, a hand-worked
8-token example, special cases that reduce to library routines, brute force
and invariants.  See each module's docstring for the passages it follows.
"""
from . import formats, indexer, brute  # noqa: F401
