"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code with the HIP library (no kernels, headers, helpers, tables
or pre/post-processing) and imports nothing from it.

What it computes, and where the pages state it:

* ``attention`` -- the exact result, ``softmax(scale * q k^T) v`` per query
  row, plus the natural-log log-sum-exp of the visible scaled scores.  The
  FlashAttention explainer (aiunderstanding.org, "Deep dive" and the FAQ
  answer on how its output compares) says the fused method produces exactly
  the values of standard attention; this function *is* standard attention,
  written as the two-pass softmax (max, then sum, then weighted sum).
* ``attention_online`` -- the same quantity via the running-max / running-sum
  recurrence that the explainer's "Technical insight" section and its FAQ
  describe (tiles arrive one by one, partial results are rescaled).  Used
  only to pin ``attention``.
* ``split_partials`` / ``merge`` / ``combine`` / ``finish`` -- the split-KV
  decode: partial (m, l, o~) per sequence chunk, merged by the associative
  log-sum-exp operator along the sequence axis in a tree, as the Tree
  Attention abstract (express24.ir page) describes for the reduction across
  the sequence axis.
* ``visibility`` -- the causal / sliding-window mask predicate.  Local
  attention ("tokens attend only to their neighbours", thread on extending
  LLM context, point 1) is a window; causal and GQA are readings stated in
  ``attention.py``.

* ``attention_backward`` (``backward.py``) -- the gradients dq, dk, dv of
  ``sum(do * attention(q, k, v))``: the derivative of the definition above,
  written out by the chain rule (the pages name training as a use but print
  no backward algorithm).  Pinned by tests/pins_backward.py (central finite
  differences of ``attention``, torch autograd, closed-form special cases).

* ``e4m3_decode`` / ``attention_fp8`` (``fp8.py``) -- the exact attention of
  fp8 (OCP E4M3) inputs with per-tensor descale factors: the inputs decoded
  to their real values, then ``attention``.  Pinned by tests/pins_fp8.py (all
  256 codes against torch's float8_e4m3fn conversion and the format's closed
  forms, descale identities).

Every function is fp64 throughout.  Parity pins: see tests/test_oracle_pins.py
(brute force, online == two-pass, split+tree == unsplit, uniform scores,
permutation invariance, special cases, overflow safety, GQA == MHA, the
energy-gradient identity, torch SDPA cross-check, hand-derived golden cases).
No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visibility,
    attention,
    attention_online,
    decode,
    split_bounds,
    split_partials,
    merge,
    combine,
    finish,
)
from .backward import attention_backward  # noqa: F401
from .fp8 import E4M3_MAX, attention_fp8, e4m3_decode  # noqa: F401
