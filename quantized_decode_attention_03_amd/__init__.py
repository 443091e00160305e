"""Low-bit KV-cache quantization and fused-dequant decode attention for MI355X.

The work runs in hand-written HIP kernels (gfx950) behind the C ABI declared in
include/kvq.h; this package is a thin ctypes binding over that library plus the
seeded synthetic workloads. Importing it loads nothing; the native library is
loaded on first use and its absence is an error (there is no CPU fallback).
"""
