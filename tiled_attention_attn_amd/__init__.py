"""MI355X (gfx950) fused tiled attention forward and in-kernel broadcast linear layer.

The computation lives in libattn.so (HIP kernels behind the C ABI declared in
include/attn.h); this package is its thin Python binding. Importing the
package does not load the library; the first call does, and fails loudly if
the library has not been built.
"""
from ._binding import (ATTN_BF16, ATTN_EINVAL, ATTN_ELAUNCH, ATTN_ESCRATCH, ATTN_EUNSUPPORTED,
                       ATTN_F32, ATTN_OK, LIB_PATH, AttnError, attn_fwd, attn_fwd_bcast, bcast_group,
                       attn_fwd_block_sparse, attn_fwd_jagged, attn_fwd_qknorm,
                       attn_fwd_qknorm_noalloc, attn_strerror, attn_version, ikbo_linear,
                       load_library)

__all__ = ["attn_fwd", "attn_fwd_bcast", "bcast_group", "attn_fwd_block_sparse", "attn_fwd_jagged",
           "attn_fwd_qknorm", "attn_fwd_qknorm_noalloc", "ikbo_linear", "attn_strerror", "attn_version", "load_library",
           "AttnError", "LIB_PATH", "ATTN_OK", "ATTN_EINVAL", "ATTN_EUNSUPPORTED",
           "ATTN_ELAUNCH", "ATTN_ESCRATCH", "ATTN_F32", "ATTN_BF16"]
