"""MI355X-native training step of the tile-based differentiable Gaussian
rasterizer: a gfx950 HIP library behind a C ABI (``include/gs.h``), a ctypes
binding with the same names (``_lib``), and a step driver (``step``).

Importing the package loads nothing; ``_lib.lib()`` loads the HIP library and
raises if it is not built.
"""
