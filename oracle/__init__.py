"""Plain, slow, fp64 CPU oracle for single-query decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers); the only thing the two sides have in
common is the seeded input generator in ``workloads``, which holds none of the
attention arithmetic.

Sources (cited by page title and section; the pages are web articles):

* "Flash Decoding" explainer (aiqz.cc), section 1 (standard attention, its
  four steps), section 2 (split-KV partials, the max rescale merge), the
  numpy demonstration, and section 3 (KV cache paged into fixed-size pages).
* "FlashDecoding" deployment blog (m.nxbn.cn), section 1 and the
  ``fixed_max_value`` / ``fallback_on_overflow`` settings of section 3 and
  troubleshooting item four of section 5 (fixed maximum with fallback).
* "Faster Than Flash" digest (longzhangge.com), sections 3 (top-delta),
  4 (pseudo-max from sink and local anchors), 5 (2-bit main part plus 8-bit
  residual) and Fig. 2 (the pipeline).

Every floating-point step is float64 unless a function says otherwise.  The
key packer (``ffd.pack_keys``) takes its integer decisions in float32 with
round-to-nearest-even, the same precision as the GPU packer, because a
quantised code is an integer decided by floating point.

Pinned by ``tests/test_oracle_*.py``; see each function for its pin.  The one
part with no pin is the pages' end-to-end sparsity / speed / quality figures,
which need trained models: parity unpinned there.
"""
from . import flash_decoding, paged, unified, ffd, append, multi_row  # noqa: F401
