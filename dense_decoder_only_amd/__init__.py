"""MI355X-native (gfx950) forward+backward training step of a nanochat-style
dense decoder.

The compute lives in ``libnc.so`` (hand-written HIP kernels behind a C ABI
declared in ``include/nc.h``); ``dense_decoder_only_amd.nc`` is the thin
ctypes binding.  Importing this package does not load the library: the
binding loads it on first use and raises if it has not been built.
"""
__version__ = "0.1.0"
