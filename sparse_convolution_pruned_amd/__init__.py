"""Native SparseConv2D for pruned ViT token sequences on AMD MI355X (gfx950).

The compute lives in the HIP/C-ABI library ``libsvconv.so`` (built from
``csrc/``); ``ops`` is the thin ctypes binding over it and ``workloads``
draws seeded synthetic inputs.  Importing the package loads nothing: the
library is opened on first use of ``ops`` and a missing or unloadable
library raises immediately -- there is no CPU fallback.
"""
__all__ = ["ops", "workloads"]
