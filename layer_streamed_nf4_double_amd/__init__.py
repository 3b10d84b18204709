"""Layer-streamed LoRA training over a frozen NF4 decoder base on MI355X.

Submodules:
  build    -- compiles liblsn.so (hipcc, gfx950) in-tree
  _lib     -- ctypes binding of include/lsn.h (same function names)
  trainer  -- SFT / DPO step loops (orchestration of C-ABI calls)

Importing ``_lib`` or ``trainer`` requires the built library; there is no
fallback implementation.
"""
__all__ = ["build", "_lib", "trainer"]
