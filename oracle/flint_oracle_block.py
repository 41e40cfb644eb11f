"""FP64 CPU oracle of the Flint attention block: projections around the layer.

TEST INFRASTRUCTURE ONLY, like the other oracle modules: only the tests, the
package's ``smoke()`` check and the CPU-baseline leg of the benchmark may import
it; the product path never does, and nothing is shared with it.

flint.layers API page, ``FlintAttention``: separate q, k and v projections,
per-head RMSNorm, selective NeoX RoPE, learned sinks, and an output projection;
``forward`` maps hidden states [tokens, hidden_size] to [tokens, hidden_size].
FlintConfig page: hidden_size 2048, 32 query heads, 4 key/value heads, head
dimension 128, no attention bias (``attention_bias`` False; discussion #26 on
RecursiveSI/flint notes that this makes fused QKV kernels trivial). A
projection is an ``nn.Linear`` without bias: y = x W^T with W [out, in].
The projected rows are read as [heads, head_dim], head-major: channel
h * head_dim + d of the projection is channel d of head h (the attention
output is laid out the same way before ``o_proj``).
"""

from __future__ import annotations

import numpy as np

from . import flint_oracle as fo

__all__ = ["linear", "flint_attention_block"]


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """nn.Linear without bias: x [.., in] times W^T, W [out, in]."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def split_heads(y: np.ndarray, head_dim: int) -> np.ndarray:
    """[T, heads * head_dim] -> [T, heads, head_dim], head-major."""
    T = y.shape[0]
    return y.reshape(T, y.shape[1] // head_dim, head_dim)


def flint_attention_block(hidden, w_q, w_k, w_v, w_o, q_norm_w, k_norm_w, sinks, cu_seqlens,
                          seqused=None, positions=None, window: int = 513, use_rope: bool = True,
                          theta: float = 1.0e6, eps: float = 1.0e-6, head_dim: int = 128,
                          rows=None):
    """Attention block forward in FP64 on hidden [T, hidden_size].

    Returns (y [len(rows), hidden_size], (q, k, v) [T, heads, head_dim] of the
    projections, o [len(rows), heads * head_dim] of the attention); rows=None is
    every token. Padded tokens attend to nothing: their attention output is 0,
    and so is their y.
    """
    q = split_heads(linear(hidden, w_q), head_dim)
    k = split_heads(linear(hidden, w_k), head_dim)
    v = split_heads(linear(hidden, w_v), head_dim)
    o = fo.flint_attention(q, k, v, q_norm_w, k_norm_w, sinks, cu_seqlens, seqused=seqused,
                           positions=positions, window=window, use_rope=use_rope, theta=theta,
                           eps=eps, rows=rows)
    o = o.reshape(o.shape[0], -1)
    return linear(o, w_o), (q, k, v), o
