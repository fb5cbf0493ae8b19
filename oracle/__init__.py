"""Plain CPU oracle for the fine-grained-scaled FP8 / FP8xFP4 GEMM path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``fp4_gemm_dense_amd`` and its HIP library) never imports, links or calls it,
and this package imports nothing from the product path: the two share no code.

Everything here is written from the pages' description of what is computed
(the DeepGEMM pages: the usage guide's "五、使用方法" for ``D = C + A @ B`` in
NT layout and the grouped forms, the Mega-MoE/FP4 news page's "FP4 精度支持"
for UE8M0 packing) and evaluated in float64 with numpy, with no blocking, fusion
or reordering beyond the plain definition of each operation.

Modules
-------
``formats``  exact decoders (e4m3fn, E2M1, UE8M0, bf16), the e4m3 encoder used by
             the FFN's in-pipeline requantisation, and bf16 rounding.
``ref``      the four reference operations: dense NT GEMM, M-grouped contiguous,
             M-grouped masked, and the FP8xFP4 expert FFN, plus per-element
             evaluators for spot checks at full size.

Pins: every function here is checked against something other than itself in
``tests/test_oracle.py`` (library decoders, exact rational brute force, closed
forms, exact power-of-two cases, invariants).  No function is "parity unpinned".
"""

from . import formats, ref  # noqa: F401
