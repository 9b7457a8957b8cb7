"""CPU oracle for sparse paged MXFP4 decode attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library and its Python
binding never do, and this package imports nothing from them: the two sides
share no kernels, helpers, tables or constants.  Their only common input is
the seeded generator in ``workloads/``, which draws random bytes and holds
none of the method's arithmetic.

Everything here is plain numpy in float64, written to be checked by eye
against the pages it follows:

* ``mxfp4``  -- page geometry, nibble packing and exact e2m1 x e8m0
  dequantisation (page *vllm.models.minimax_m3.amd.ops.mxfp4_pages*:
  module docstring and ``mxfp4_page_views``).
* ``decode`` -- query positions, index scores, top-k selection and GQA
  attention over the selected (or all valid) tokens.

Every function is pinned by ``tests/test_oracle_*.py`` against facts that do
not come from the oracle itself (the printed geometry, closed forms, library
routines, brute force).  Functions without such a pin say "parity unpinned"
in their docstring; at present there are none.
"""

from . import decode, mxfp4  # noqa: F401
