"""dense_gemm_row_amd: dense row-major GEMM for AMD MI355X (gfx950).

The compute path is the C-ABI shared library ``libgemm.so`` built from
``csrc/``; :mod:`dense_gemm_row_amd.gemm` is its thin ctypes binding.
"""
