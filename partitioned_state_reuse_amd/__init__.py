"""Partitioned DiT self-attention with selective attention-state reuse, for MI355X (gfx950).

The hot path (partition attention with state-cache update, LSE-weighted state merge,
partition importance, local-state-change reduction) runs in the HIP library
`libdit_attn.so` behind the C ABI of include/dit_attn.h; the group planner is host C++ in
the same library.  `api` is the Python binding (ctypes; PyTorch for memory and streams).

Importing the package does not load the library; the first call does, and raises if the
library has not been built (partitioned_state_reuse_amd/build.py).
"""
__all__ = ["api", "build"]
