"""MI355X-native TARA dense and pooled block-sparse attention.

The compute path is the HIP library ``libh3attn.so`` built from ``csrc/`` for
gfx950 (``python -m block_sparse_attention_02_amd.build``); the submodule
``api`` marshals arguments to its C entry points and loads the library on
first use. ``workloads`` holds the seeded synthetic inputs.
"""
__all__ = ["api", "workloads", "build"]
