"""MI355X-native verification attention for long-context speculative decoding.

Submodules:
  ssverify   ctypes binding of the C-ABI library libssverify.so (loaded on
             first use; raises if the library is missing)
  workloads  seeded synthetic inputs shaped like the verification workloads
  build      compiles the HIP library for gfx950
"""
