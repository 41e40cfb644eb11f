"""Shared test helpers: workload conversion and oracle invocation."""

from __future__ import annotations

import numpy as np
import torch

from oracle import flint_attention


def f64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.to(torch.float64).numpy()
    return np.asarray(t, np.float64)


def i64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.to(torch.int64).numpy()
    return np.asarray(t, np.int64)


def oracle_for(wl, layer, rows=None, debug=False, **over):
    """Run the oracle on a workload and one of its layers."""
    args = dict(q=f64(wl.q), k=f64(wl.k), v=f64(wl.v), q_norm_w=f64(wl.q_norm_w),
                k_norm_w=f64(wl.k_norm_w), sinks=f64(wl.sinks), cu_seqlens=i64(wl.cu_seqlens),
                seqused=i64(wl.seqused), positions=i64(wl.positions), window=layer.window,
                use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps, rows=rows, debug=debug)
    args.update(over)
    return flint_attention(**args)


def seq_index(cu, T):
    """(sequence id, index in sequence) of every token."""
    cu = np.asarray(cu, np.int64)
    t = np.arange(T)
    s = np.searchsorted(cu, t, side="right") - 1
    return s, t - cu[s]
