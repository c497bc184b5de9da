"""One tensor-parallel rank's share of a transformer MLP on MI355X (gfx950).

The compute lives in ``libtpmlp.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tp_mlp.h``).  ``binding`` wraps that ABI with the same
entry-point names; ``configs`` and ``synth`` describe and draw the workloads.

The binding is imported lazily so that the shape tables and the input
generator can be used on a machine where the library has not been built.
"""
from __future__ import annotations


def __getattr__(name):
    # every entry point (tp_*), constant (TP_*) and helper of the binding
    if name.startswith(("tp_", "TP_")) or name in ("binding", "TPError", "load_library",
                                                    "ABI_FUNCTIONS"):
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
