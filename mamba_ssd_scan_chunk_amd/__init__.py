"""MI355X-native Mamba-2 SSD layer scan: chunked prefill and O(1) cached decode.

The compute lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/ssd.h``).  ``binding`` is a thin
ctypes layer over it; ``synth`` draws seeded synthetic inputs.
"""
