"""MI355X-native hyper-connection residual-stream layer (mHC and xHC).

The layer runs in ``libxhc.so`` (hand-written HIP kernels for gfx950 behind
the C ABI in ``include/xhc.h``); ``binding`` is its ctypes binding and
``synth`` the seeded synthetic workload generator.
"""
__all__ = ["binding", "synth", "build"]
