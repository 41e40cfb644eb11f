"""FP64 CPU oracle of the Flint sink-aware attention backward.

TEST INFRASTRUCTURE ONLY, like the forward oracle next to it: only the tests,
the package's ``smoke()`` check and the CPU-baseline leg of the benchmark may
import it; the product path never does, and nothing is shared with it.

The layer is the forward of ``flint_oracle`` (same page citations): per-head
weight-form RMSNorm of q and k, NeoX RoPE on sliding layers, logits
q'.k'/sqrt(D), a zero-value per-head sink logit in the softmax, grouped-query
attention. For a loss L with upstream gradient dO = dL/dO this module writes
out the chain rule step by step, per sequence and head, over whole rows:

  forward by-products   W = softmax weights, p = sink weight,
                        lse = log(exp(sink) + sum_j exp(z_j)), O = W V
  row term              Dr_t = dO_t . O_t
  softmax               dW = dO V^T,  dZ = W * (dW - Dr)
                        (the sink column has value 0, so its dW is 0 and
                        dL/dsink_h = -sum_t p_t Dr_t: the sink adjoint)
  values                dV_j = sum_t W_tj dO_t
  logits                dq'_t = sum_j dZ_tj k'_j / sqrt(D),
                        dk'_j = sum_t dZ_tj q'_t / sqrt(D)
  RoPE                  a rotation by angle pos*omega; its adjoint is the
                        rotation by -pos*omega
  RMSNorm (weight form) y = x r w with r = 1/sqrt(mean(x^2) + eps):
                        dw = sum over tokens and heads of dy * x r,
                        dx = r (dy w - (x r) mean(x r * dy w))
  GQA                   dk', dv of kv head g sum over its query heads.

The backward is what the pages' training recipes need (discussion #26 on
RecursiveSI/flint, section "Where other stacks fail": sinks in backward, and
the sink gradient). Padded tokens get zero gradients: they take no part in
the layer (flint.layers page, FlintAttention.forward).

Row sampling: ``rows`` selects the dq rows and ``keys`` the dk/dv rows to
compute; the row statistics (lse, Dr) always cover every valid row, since a
key's gradient needs every query that sees it. The weight gradients need every
row and key and are returned only when both selections are None.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import flint_oracle as fo

__all__ = ["flint_attention_backward"]


def _rope_adjoint(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Adjoint (= inverse) of the RoPE rotation: the rotation by the opposite angle."""
    return fo.rope_neox(x, -np.asarray(pos, np.float64), theta)


def _logit_scale(head_dim: int) -> float:
    """z = q'.k' times this: 1/sqrt(D)."""
    return 1.0 / math.sqrt(head_dim)


def _softmax_backward(W: np.ndarray, dW: np.ndarray, Dr: np.ndarray) -> np.ndarray:
    """dZ = W * (dW - Dr): the softmax Jacobian applied to dW, with Dr = sum_j W_j dW_j."""
    return W * (dW - Dr[:, None])


def _sink_adjoint(p: np.ndarray, Dr: np.ndarray) -> float:
    """dL/dsink = p * (0 - Dr) summed over rows: the sink's value is 0."""
    return -float(np.sum(p * Dr))


def _rms_norm_backward(x: np.ndarray, w: np.ndarray, eps: float, dy: np.ndarray):
    """Backward of y = x / sqrt(mean(x^2) + eps) * w over the last axis.

    Returns (dx, dw_terms) where dw_terms = dy * x r is summed by the caller
    over every token and head that shares the weight.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xn = x * r
    dyw = dy * w
    dx = r * (dyw - xn * np.mean(xn * dyw, axis=-1, keepdims=True))
    return dx, dy * xn


def flint_attention_backward(q, k, v, q_norm_w, k_norm_w, sinks, cu_seqlens, dout,
                             seqused=None, positions=None, window: int = 513,
                             use_rope: bool = True, theta: float = 1.0e6, eps: float = 1.0e-6,
                             rows=None, keys=None) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of the sink-aware attention layer in FP64.

    Arguments as ``flint_attention`` plus dout [T, H, D] = dL/dO. Returns a dict:
      dq [len(rows), H, D], dk [len(keys), G, D], dv [len(keys), G, D]
        (rows / keys None = every token),
      dsink [H] (always complete: it needs only row statistics),
      dq_norm_w, dk_norm_w [D] (None unless rows and keys are both None),
      out [T, H, D] and lse [T, H] of the forward (lse = -inf on padded rows).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    qw_ = np.asarray(q_norm_w, np.float64)
    kw_ = np.asarray(k_norm_w, np.float64)
    sinks = np.asarray(sinks, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, H, D = q.shape
    G = k.shape[1]
    n = len(cu) - 1
    inv_sqrt_d = _logit_scale(D)
    pos_all = None if positions is None else np.asarray(positions, np.int64)
    full = rows is None and keys is None
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    keys = np.arange(T, dtype=np.int64) if keys is None else np.asarray(keys, np.int64)

    out = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    Dr = np.zeros((T, H))
    dsink = np.zeros(H)
    dq_p = np.zeros((T, H, D))  # dL/dq' of the rows that are computed
    dk_p = np.zeros((T, G, D))  # dL/dk'
    dv = np.zeros((T, G, D))
    need_q = np.zeros(T, bool)
    need_q[rows] = True
    need_k = np.zeros(T, bool)
    need_k[keys] = True

    for s in range(n):
        start, end = int(cu[s]), int(cu[s + 1])
        L = end - start
        u = L if seqused is None else min(int(np.asarray(seqused)[s]), L)
        if u <= 0:
            continue
        idx = np.arange(u, dtype=np.int64)
        p = idx if pos_all is None else pos_all[start:start + u]
        qh = fo.rms_norm(q[start:start + u], qw_, eps)
        kh = fo.rms_norm(k[start:start + u], kw_, eps)
        if use_rope:
            qh = fo.rope_neox(qh, p, theta)
            kh = fo.rope_neox(kh, p, theta)
        vv = v[start:start + u]
        do = dout[start:start + u]
        nb = fo._row_block_size(u, H)

        # Pass 1, every valid row: softmax weights over the whole key set, the
        # output, lse and the row term Dr; the sink adjoint.
        for b0 in range(0, u, nb):
            lq = idx[b0:b0 + nb]
            A = fo.allowed_keys(lq, idx, u, window)
            for h in range(H):
                g = fo.kv_head_of(h, H, G)
                z = np.where(A, (qh[lq, h, :] @ kh[:, g, :].T) * inv_sqrt_d, -np.inf)
                W, ps, m, E = fo.sink_softmax(z, sinks[h])
                o = W @ vv[:, g, :]
                t = start + lq
                out[t, h, :] = o
                with np.errstate(divide="ignore"):
                    lse[t, h] = np.where(E > 0, m + np.log(np.where(E > 0, E, 1.0)), -np.inf)
                Dr[t, h] = np.sum(do[lq, h, :] * o, axis=-1)
                dsink[h] += _sink_adjoint(ps, Dr[t, h])

        def weights(lq, lk, h, g):
            """Softmax weights W[lq, lk] of head h from the row lse (0 where not allowed)."""
            A = fo.allowed_keys(lq, lk, u, window)
            z = (qh[lq, h, :] @ kh[lk, g, :].T) * inv_sqrt_d
            ls = lse[start + lq, h][:, None]
            with np.errstate(invalid="ignore", over="ignore"):
                return np.where(A & np.isfinite(ls), np.exp(np.where(A, z, 0.0) - ls), 0.0)

        # Pass 2a: dq' of the selected rows, each over its whole key set.
        sel_q = idx[need_q[start:start + u]]
        for b0 in range(0, len(sel_q), nb):
            lq = sel_q[b0:b0 + nb]
            for h in range(H):
                g = fo.kv_head_of(h, H, G)
                W = weights(lq, idx, h, g)
                dW = do[lq, h, :] @ vv[:, g, :].T
                dZ = _softmax_backward(W, dW, Dr[start + lq, h])
                dq_p[start + lq, h, :] = (dZ @ kh[:, g, :]) * inv_sqrt_d

        # Pass 2b: dk' and dv of the selected keys, each over every query that
        # sees it (queries after it within the window).
        sel_k = idx[need_k[start:start + u]]
        for b0 in range(0, len(sel_k), nb):
            lk = sel_k[b0:b0 + nb]
            q_hi = u if window == 0 else min(u, int(lk.max()) + window)
            lq = np.arange(int(lk.min()), q_hi, dtype=np.int64)
            for h in range(H):
                g = fo.kv_head_of(h, H, G)
                W = weights(lq, lk, h, g)
                dW = do[lq, h, :] @ vv[lk, g, :].T
                dZ = _softmax_backward(W, dW, Dr[start + lq, h])
                dk_p[start + lk, g, :] += (dZ.T @ qh[lq, h, :]) * inv_sqrt_d
                dv[start + lk, g, :] += W.T @ do[lq, h, :]

    # RoPE and RMSNorm backward, token by token (padded tokens stay zero).
    valid = np.zeros(T, bool)
    posv = np.zeros(T, np.int64)
    for s in range(n):
        start, end = int(cu[s]), int(cu[s + 1])
        u = (end - start) if seqused is None else min(int(np.asarray(seqused)[s]), end - start)
        valid[start:start + max(u, 0)] = True
        posv[start:end] = np.arange(end - start) if pos_all is None else pos_all[start:end]
    dq = np.zeros((T, H, D))
    dk = np.zeros((T, G, D))
    dq_norm_w = np.zeros(D)
    dk_norm_w = np.zeros(D)
    tq = np.nonzero(valid & need_q)[0]
    tk = np.nonzero(valid & need_k)[0]
    dqw = _rope_adjoint(dq_p[tq], posv[tq], theta) if use_rope else dq_p[tq]
    dkw = _rope_adjoint(dk_p[tk], posv[tk], theta) if use_rope else dk_p[tk]
    dq[tq], terms_q = _rms_norm_backward(q[tq], qw_, eps, dqw)
    dk[tk], terms_k = _rms_norm_backward(k[tk], kw_, eps, dkw)
    dq_norm_w += terms_q.reshape(-1, D).sum(axis=0)
    dk_norm_w += terms_k.reshape(-1, D).sum(axis=0)
    dv[~valid] = 0.0

    return {
        "dq": dq[rows],
        "dk": dk[keys],
        "dv": dv[keys],
        "dsink": dsink,
        "dq_norm_w": dq_norm_w if full else None,
        "dk_norm_w": dk_norm_w if full else None,
        "out": out,
        "lse": lse,
    }
