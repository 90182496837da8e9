"""LightningIndexer forward pass for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/li.h``); :mod:`.binding` mirrors its entry
points for Python and :mod:`.indexer` wraps them for torch tensors. Importing
this package does not load the library; the first call that needs it does,
and fails loudly if it has not been built.
"""
__version__ = "0.1.0"
