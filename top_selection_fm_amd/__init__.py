"""MI355X (gfx950) compressed-key indexer: scoring and selection of compressed KV entries.

The compute path is the C-ABI library ``libfm.so`` (hand-written HIP kernels, declared in
``include/fm.h``).  ``top_selection_fm_amd.api`` is a thin ctypes binding over it that only
marshals torch tensors into pointers; ``workloads`` builds seeded synthetic inputs.  Importing
the package loads nothing: the library is opened on first use and raises if it is missing.
"""
__all__ = ["api", "workloads"]
