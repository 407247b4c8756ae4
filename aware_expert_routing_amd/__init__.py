"""Decode-time MoE layer with batch-aware expert selection for MI355X (gfx950).

The compute path is the HIP library libmoe_decode.so (C ABI in
include/moe_decode.h); `_lib` is its ctypes binding and `workloads` draws the
seeded synthetic inputs. Importing this package loads nothing; the library is
loaded on first use and a missing build raises.
"""
__all__ = ["_lib", "workloads"]
