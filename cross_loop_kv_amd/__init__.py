"""MI355X (gfx950) library for lazy looped-Transformer inference.

``cross_loop_kv_amd.binding`` wraps the C ABI of ``liblooped_kv.so`` (declared in
include/looped_kv.h); ``cross_loop_kv_amd.inputs`` generates seeded synthetic
inputs; ``cross_loop_kv_amd.build`` compiles the HIP sources for gfx950.
The binding is imported on demand so that input generation works without the
library.
"""
__all__ = ["binding", "inputs", "build"]
