"""MI355X (gfx950) token-tree attention and token-tree verification.

The compute path is the C library libtreeverify.so (include/tree_verify.h),
built from csrc/ by `python -m tree_verification_amd.build`; `binding` wraps
it for torch tensors.  `workloads` draws the seeded synthetic inputs.

Importing this package does not load the library; the first binding call does,
and raises if it has not been built.
"""
from .binding import (kv_compact_accepted, load_library, tree_attn_forward,  # noqa: F401
                      tree_verify_greedy, tree_verify_stochastic)
