"""CPU oracle for the block-sparse attention forward -- test infrastructure.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
it.  The product path never does: it shares no code with the HIP library.
"""
from .oracle import (BLOCK, Geometry, Route, attend_block, attended_pairs, attention,  # noqa: F401
                     block_lists, block_scores, build_c, default_scale32, dense_attention,
                     densities, geometry, pool_keys, pool_queries, route, select_blocks,
                     tie_list)
