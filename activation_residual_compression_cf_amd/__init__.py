"""CompactFusion step-wise activation residual compression with sender-side error
feedback, as HIP kernels for MI355X (gfx950) behind a C ABI (``include/cf.h``).

``cf`` is the Python binding (ctypes); importing it requires the built ``libcf.so``.
"""
