"""STILL intra-layer hybrid attention on AMD Instinct MI355X (gfx950).

``hybrid_sparse_softmax_amd.still`` is the Python binding of the C-ABI
library ``libstill.so`` (``include/still.h``); ``hybrid_sparse_softmax_amd.build``
compiles it with hipcc.
"""
