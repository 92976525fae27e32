"""MI355X-native exact attention (forward + backward) behind a C-ABI library.

Submodules:
  inputs  seeded synthetic inputs (no attention arithmetic)
  fa      thin ctypes binding to the HIP library (loaded on import; raises if
          the library is not built)
  build   compiles the HIP library for gfx950
"""
