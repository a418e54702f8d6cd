"""Independent CPU oracle for the DP / Split-K / Stream-K GEMM.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import anything in this package; the library
(``dense_gemm_work_amd``) never does, and this package imports nothing from it.

* ``oracle.gemm``     -- fp64 reference GEMM over the dtype-rounded operands
                         (plain C, ``ref_gemm.c``) and the K-scaled tolerance.
* ``oracle.schedule`` -- CPU schedule simulator: wave arithmetic, unit ranges,
                         segment/role lists, owner/peer lists, coverage, the
                         decomposition heuristic and the unit cost model.
"""
