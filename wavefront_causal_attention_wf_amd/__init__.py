"""MI355X-native (gfx950) wave-tick attention for chunk-wise causal wavefront
generation.

The compute path lives in a C-ABI shared library (libwfattn.so, declared in
include/wf_attn.h) built from csrc/ with hipcc. `wfattn` is the thin Python
binding over it; importing `wfattn` loads the library and raises if it has not
been built. `inputs` draws the seeded synthetic workloads.
"""
__all__ = ["inputs"]
