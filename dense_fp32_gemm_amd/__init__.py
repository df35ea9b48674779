"""dense_fp32_gemm_amd -- dense FP32 GEMM for AMD MI355X (gfx950, CDNA4).

C[M x N] = A[M x K] . B[K x N], row-major, any M/N/K, computed by hand-written
HIP kernels on the FP32 matrix cores behind the C-ABI library
``libgemm_f32.so`` (declared in ``include/gemm_f32.h``).  ``binding`` is the
ctypes layer with the same names; ``inputs`` holds the seeded operand
generators.  The binding loads the library on first use.
"""
