"""MI355X-native indexer top-k selection with fused paged slot mapping.

The work runs in hand-written gfx950 HIP kernels behind the C ABI declared in
include/sparse_topk.h; ``sparse_attention_indexer_amd.topk`` is the ctypes
binding (torch supplies device memory and streams). Importing the package does
not load the library; the first call does, and raises if it is not built.
"""

__all__ = ["topk"]
