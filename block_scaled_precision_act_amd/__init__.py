"""MI355X (gfx950) block-scaled low-precision linear layer: MXFP4 A4W4 and PTPC FP8 A8W8.

The compute path is the C-ABI library ``libmxgemm.so`` (hand-written HIP
kernels); ``mxgemm`` is its thin ctypes binding and ``synth`` the seeded
input generators.  Importing the package loads nothing; the first call into
``mxgemm`` loads the library and raises if it has not been built.
"""
__all__ = ["mxgemm", "synth"]
