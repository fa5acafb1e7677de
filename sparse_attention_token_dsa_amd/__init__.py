"""MI355X (gfx950) DSA lightning-indexer selector: DSA, MISA and HISA.

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libsaindexer.so``, declared in ``include/sa_indexer.h``).  The binding in
``sparse_attention_token_dsa_amd.api`` only marshals torch tensors into that
ABI; it is loaded on first use.
"""
__all__ = ["api", "synth"]
