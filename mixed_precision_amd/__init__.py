"""MI355X-native routed FP16/INT8 prefill attention (TileMix hot path).

The computation lives in the HIP library ``libtilemix.so`` (C ABI in
``include/tilemix.h``); ``mixed_precision_amd.tilemix`` is its thin ctypes
binding.  Build with ``__graft_entry__.build()``.
"""
__all__ = ["tilemix"]
