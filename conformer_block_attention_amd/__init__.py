"""MI355X-native block-local multi-head self-attention (Granite-Speech conformer encoder).

The compute path is libgsattn.so (HIP kernels for gfx950, C ABI in
include/gsattn.h); `gsattn` is its Python binding.  Importing this package
does not load the library; the first call does, and fails loudly if the
library has not been built.
"""
__all__ = ["gsattn", "workloads", "accounting"]
