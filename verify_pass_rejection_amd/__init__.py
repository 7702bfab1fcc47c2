"""MI355X-native verify step of speculative decoding.

The hot path (verify attention over the draft positions, chain rejection
sampling, greedy tree acceptance) runs in hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/spec_verify.h``.  This package holds the
kernels' sources (``csrc/``), the thin ctypes binding (``native``) and the
seeded synthetic workloads (``inputs``).
"""
