"""MI355X (gfx950) gated delta rule: HIP kernels behind a C ABI (libgdn.so).

The binding in ``gdn`` loads the library on first use and raises if it is
missing; there is no CPU fallback.
"""
