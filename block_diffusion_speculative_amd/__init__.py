"""MI355X (gfx950) native DFlash draft-and-verify step.

Submodules:
  configs  -- named workloads (shapes only)
  inputs   -- seeded synthetic inputs (no arithmetic of the method)
  _lib     -- ctypes binding of libdflash.so (include/dflash.h)
  engine   -- device-resident drafter state and the three step calls

The HIP library is loaded lazily on first use; importing this package does
not touch the GPU.
"""
__all__ = ["configs", "inputs"]
