"""MI355X (gfx950) Sol-Attn block-sparse attention forward.

The kernels live in libsol.so (C ABI: include/sol.h); ``sol`` is the ctypes
binding over it.  Importing the package loads libsol.so and raises ImportError
when it has not been built.
"""
from .sol import (BLOCK, NOALLOC_SCRATCH_BYTES, SOL_ERR_SCRATCH, Desc, SolError, attn, attn_dense, default_scale, forward,  # noqa: F401
                  gate, make_desc, num_blocks, packed_offsets,
                  qk_norm_rope_pool, route, route_noalloc, route_outputs, route_pooled,
                  route_workspace_bytes, status_str)
