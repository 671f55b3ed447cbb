"""MI355X-native CSA2 (Compressed Sparse Attention 2) hot path.

The work runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/csa2.h``, built into ``libcsa2.so`` next to this file).  The Python
side only marshals arguments: see ``sparse_long_context_csa2_amd.binding``.
``synth`` draws the seeded synthetic inputs.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in ("binding", "synth"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
