"""MI355X (gfx950) all-reduce core: the rank-partial sum and the sum fused
with bias, residual and RMSNorm, as hand-written HIP kernels behind a C ABI.

The binding (``ar``) loads ``libar.so`` on first use; importing this package
does not touch the GPU.
"""
