"""MI355X-native MoE expert-parallel dispatch / combine (DeepEP-style token exchange).

The hot path -- dispatch layout, dispatch (with fused BF16->FP8 e4m3 pack),
combine (fp32 weighted gather-reduce to BF16) and the backward pair -- runs in
hand-written HIP kernels for gfx950 behind the C ABI declared in include/ep.h.

Submodules:
  ep         ctypes binding of libep.so (same names as the C ABI) plus a small
             torch-tensor convenience wrapper (argument marshalling only)
  workloads  seeded synthetic inputs (routing, activations, gradients)
  build      compiles libep.so with hipcc for gfx950

Nothing is loaded at import time; ``ep.load()`` raises if libep.so is missing.
"""
__all__ = ["ep", "workloads", "build"]
