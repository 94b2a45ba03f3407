"""MI355X-native per-frame decode hot path of a MiniMax-Music-3-style audio LM.

- ``m3``      : Python binding of the libm3 C ABI (include/m3.h), same names.
- ``runtime`` : packs a model's weights on the GPU and drives whole frames.
- ``configs`` : model shapes; ``synth``: seeded synthetic inputs.
- ``build``   : compiles libm3.so (hipcc, gfx950) in-tree.
"""
__version__ = "0.1.0"
