"""MI355X-native time-domain SAR backprojection.

The computation lives in the HIP library ``libsarbp.so`` (C ABI: include/sarbp.h);
:mod:`domain_backprojection_amd.sarbp` is its ctypes binding.  Importing the
binding fails loudly when the library has not been built.
"""
__all__ = ["sarbp"]
