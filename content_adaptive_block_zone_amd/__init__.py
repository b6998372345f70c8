"""Prism content-adaptive block-sparse video attention on MI355X (gfx950).

The computation lives in libprism.so (HIP kernels behind a C ABI, include/prism.h);
`api` binds each C call under the same name, `pipeline.PrismLayer` sequences them for
one attention layer.  Build the library with `python -m content_adaptive_block_zone_amd.build`.
"""
