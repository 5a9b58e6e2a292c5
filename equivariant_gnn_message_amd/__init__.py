"""MI355X-native equivariant message-passing convolution.

``e3conv`` is the ctypes binding of the C-ABI library ``libe3conv.so`` (HIP
kernels for gfx950 plus the host-side plan builder); ``synth`` draws seeded
synthetic workloads.  Importing the package does not load the library; the
first use of ``e3conv`` does, and raises if it is missing.
"""
