"""paged_kv_attention_15_amd -- MI355X (gfx950) paged-KV attention.

The product is libpkv.so (HIP kernels behind the C ABI in include/pkv.h); the
`pkv` module is its ctypes binding and `workloads` draws seeded synthetic
inputs.  Importing the package loads nothing: the library is loaded on the
first call into `pkv`, and that call fails loudly when it has not been built.
"""
__all__ = ["pkv", "workloads"]
