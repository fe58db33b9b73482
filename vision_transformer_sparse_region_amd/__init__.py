"""MI355X (gfx950) Bi-Level Routing Attention forward.

The compute path is libbra.so (HIP kernels behind a C ABI, include/bra.h);
`vision_transformer_sparse_region_amd.bra` is its ctypes binding.  Importing
this package loads nothing; `bra` loads the library on first use and raises
if it has not been built.
"""
