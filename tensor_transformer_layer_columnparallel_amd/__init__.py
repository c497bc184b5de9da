"""One tensor-parallel rank's share of a transformer MLP on MI355X (gfx950).

The compute lives in ``libtpmlp.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tp_mlp.h``).  ``binding`` wraps that ABI with the same
entry-point names; ``configs`` and ``synth`` describe and draw the workloads.

The binding is imported lazily so that the shape tables and the input
generator can be used on a machine where the library has not been built.
"""
from __future__ import annotations

_ABI_NAMES = (
    "tp_column_linear",
    "tp_row_linear",
    "tp_mlp_shard_fwd",
    "tp_mlp_shard_bwd",
    "tp_shard_reduce",
    "tp_status_string",
)


def __getattr__(name):
    if name in _ABI_NAMES or name in ("binding", "TPError", "load_library"):
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
