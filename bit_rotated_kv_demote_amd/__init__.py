"""MI355X-native OSCAR-style 2-bit KV demotion and tiered decode attention.

The compute path is the HIP library ``libamdoscar.so`` (built from
``csrc/``) behind the C ABI in ``include/oscar.h``; ``binding`` marshals
arguments to it.  Importing this package does not load the library.
"""
