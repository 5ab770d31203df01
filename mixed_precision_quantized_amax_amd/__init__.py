"""MI355X (gfx950) MixQ-style mixed-precision linear layer.

``mixq`` holds the binding of the HIP library ``libmixq.so`` (C ABI in
``include/mixq.h``); ``workloads`` holds the seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use.
"""
__all__ = ["mixq", "workloads", "build"]
