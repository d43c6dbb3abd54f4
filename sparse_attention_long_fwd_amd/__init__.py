"""MI355X-native (gfx950) forward pass of VideoNSA's hybrid attention layer.

Text rows keep dense causal attention; video rows go through Native Sparse
Attention: a compression branch over block tokens, a selection branch over the
top-n blocks per GQA group (scored from the compression probabilities) and a
sliding-window branch, mixed per head by gates.  All arithmetic runs in the HIP
kernels of ``libnsa.so`` behind the C ABI of ``include/nsa.h``; ``nsa`` is the
ctypes binding.
"""
from . import nsa  # noqa: F401
from .nsa import (nsa_cmp_attn_scores, nsa_compress_kv, nsa_hybrid_layer_fwd,  # noqa: F401
                  nsa_hybrid_layer_workspace_size, nsa_sparse_attn_fwd, nsa_sparse_attn_workspace_size,
                  nsa_topk_blocks)
