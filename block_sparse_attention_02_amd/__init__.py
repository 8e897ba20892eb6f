"""MI355X-native TARA dense and pooled block-sparse attention.

The compute path is the HIP library ``libh3attn.so`` built from ``csrc/`` for
gfx950; ``api`` marshals arguments to its C entry points. ``workloads`` holds
the seeded synthetic inputs.
"""
__all__ = ["workloads", "api"]


def __getattr__(name):
    if name == "api":
        from . import api
        return api
    raise AttributeError(name)
