"""CPU oracle for the fp16 "TN" GEMM and its fragment layouts.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, header, table or constant generator with the HIP
implementation in ``mma_fragment_layouts_tn_amd``.

Contents
--------
``layout``   plain shape:stride evaluator (nested tuples, first-mode-fastest
             decode), composition and right inverse as brute-force tables,
             the closed-form thread/value maps the pages print for the SM80
             atoms, a model of TiledMMA partitioning, the ldmatrix.x4 route
             rule, and closed-form gfx950 MFMA operand maps.
``fp16``     exact IEEE-754 binary16 decode, round-to-nearest-even encode,
             and the fp16 ulp used by the tolerances.
``gemm``     the float64 reference D(m,n) = C(m,n) + sum_k A(m,k) B(n,k)
             (plain C triple loop via ctypes, plus a pure-Python version
             for tiny shapes).
``compare``  the acceptance rules (bit-exact on integer-valued inputs,
             1e-4*sqrt(K) absolute for fp32 output, +1 fp16 ulp for fp16).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms or library routines, except
the gfx950 MFMA operand maps, which the pages do not cover ("parity unpinned"
on the CPU; the GPU probe test pins them against the hardware).
"""
