"""FP64 CPU oracle of the Flint sink-aware attention forward (prefill).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's ``smoke()`` check and
the CPU-baseline leg of the benchmark may import this module. The product path
(the HIP library and its Python binding) never calls it, and it shares no code,
table or constant generator with that path.

It is the plain definition of the layer written out in NumPy float64, one
query row at a time in meaning (rows are only batched for speed; every row is
computed over its whole key set with no online or blocked softmax):

  1. per-head RMSNorm of q and k in weight form, eps inside the square root
     ("flint" model page of NeMo AutoModel, section "Model Architecture":
     query/key normalization precedes RoPE; Hugging Face discussion #26 on
     RecursiveSI/flint, "What was unusually easy": plain RMSNorm times w, not
     the 1+w variant; FlintConfig API page: rms_norm_eps = 1e-06);
  2. on sliding layers only, NeoX RoPE on all 128 channels, channel c turning
     with channel c+64 ("Model Architecture"; flint.layers API page,
     ``FlintAttention._apply_rope``: corresponding channels in the two halves);
  3. the allowed key set: same sequence, not padding, causal, and within the
     window of W keys that counts the current token (W = 513: the current token
     and 512 before it, "Model Architecture"; discussion #26, "Configuration
     oddities" item 4); W = 0 is full causal attention (flint.layers page,
     ``FlintAttention.forward``);
  4. logits q.k / sqrt(head_dim) and a per-query-head FP32 sink logit that
     enters the max and the denominator with zero value, is not a token, and is
     not scaled (discussion #26, "What was unusually easy" and "Configuration
     oddities" item 5; flint.layers page, ``_FlintSinkParameters``);
  5. grouped-query attention: 32 query heads over 4 key/value heads, query head
     h reading key/value head h // 8 ("Model Architecture").

Padded query rows (index in sequence >= valid length) output exactly zero: the
flint.layers page says padded queries and keys leave real attention and only
the zero-value sink stays valid. A row whose sink is -inf and whose key set is
empty also outputs zero (0/0 taken as 0).
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "rms_norm",
    "rope_neox",
    "rope_frequencies",
    "kv_head_of",
    "allowed_keys",
    "sink_softmax",
    "flint_attention",
]


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Weight-form RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_c = theta^(-2c/head_dim) for c in [0, head_dim/2) (default RoPE type)."""
    c = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * c / head_dim)


def rope_neox(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate channel c with channel c + D/2 by angle pos * omega_c.

    x is [N, heads, D] and pos is [N] (integer positions).
    """
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, np.float64)[:, None] * rope_frequencies(x.shape[-1], theta)[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def kv_head_of(h, num_q_heads: int, num_kv_heads: int):
    """Key/value head read by query head h: contiguous groups of H/G heads."""
    return h // (num_q_heads // num_kv_heads)


def allowed_keys(lq: np.ndarray, lk: np.ndarray, valid_len: int, window: int) -> np.ndarray:
    """Boolean [len(lq), len(lk)]: key index lk is allowed for query index lq.

    Indices are positions inside one sequence. A key is allowed when it is not
    padding, not after the query, and (window > 0) at most window-1 before it.
    """
    lq = np.asarray(lq, np.int64)[:, None]
    lk = np.asarray(lk, np.int64)[None, :]
    ok = (lk < valid_len) & (lk <= lq)
    if window > 0:
        ok &= (lq - lk) <= (window - 1)
    return ok


def sink_softmax(z: np.ndarray, sink: np.ndarray):
    """Softmax over [sink, z...] along the last axis, the sink column dropped.

    z is [..., K] with -inf at disallowed keys; sink broadcasts to z[..., 0].
    Returns (weights [..., K], p_sink [...], m [...], E [...]). With every
    entry -inf (sink included) the weights and p_sink are 0.
    """
    sink = np.broadcast_to(np.asarray(sink, np.float64), z.shape[:-1])
    zmax = np.max(z, axis=-1) if z.shape[-1] else np.full(z.shape[:-1], -np.inf)
    m = np.maximum(sink, zmax)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(invalid="ignore"):
        e = np.exp(z - m_safe[..., None])
        es = np.exp(sink - m_safe)
    E = es + np.sum(e, axis=-1)
    inv = np.where(E > 0, 1.0 / np.where(E > 0, E, 1.0), 0.0)
    return e * inv[..., None], es * inv, m, E


def _row_block_size(n_keys: int, heads: int) -> int:
    budget = 1 << 23  # elements of the [rows, heads, keys] logit block
    return max(1, min(256, budget // max(1, heads * max(n_keys, 1))))


def flint_attention(q, k, v, q_norm_w, k_norm_w, sinks, cu_seqlens, seqused=None,
                    positions=None, window: int = 513, use_rope: bool = True,
                    theta: float = 1.0e6, eps: float = 1.0e-6, rows=None,
                    debug: bool = False):
    """Sink-aware grouped-query attention forward in FP64.

    Arguments (arrays are converted to float64 / int64 losslessly):
      q [T, H, D], k [T, G, D], v [T, G, D]; q_norm_w, k_norm_w [D];
      sinks [H] in natural-log units; cu_seqlens [n+1]; seqused [n] or None
      (valid prefix length per sequence); positions [T] or None (then the
      index inside the sequence); window W (0 = full causal); use_rope; theta;
      eps; rows: token indices to compute (None = all).
    Returns O [len(rows), H, D] float64, and with ``debug`` also a dict of
    per-row ``weights`` [rows, H, Lmax] indexed by key position in the
    sequence, ``p_sink``, ``m`` and ``E`` [rows, H].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sinks = np.asarray(sinks, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    T, H, D = q.shape
    G = k.shape[1]
    n = len(cu) - 1
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), H, D), np.float64)
    lens = cu[1:] - cu[:-1]
    Lmax = int(lens.max()) if n > 0 else 0
    dbg: Optional[Dict[str, np.ndarray]] = None
    if debug:
        dbg = {"weights": np.zeros((len(rows), H, Lmax)), "p_sink": np.zeros((len(rows), H)),
               "m": np.full((len(rows), H), -np.inf), "E": np.zeros((len(rows), H))}
    pos_all = None if positions is None else np.asarray(positions, np.int64)
    order = np.argsort(rows, kind="stable")
    srows = rows[order]
    for s in range(n):
        start, end = int(cu[s]), int(cu[s + 1])
        L = end - start
        u = L if seqused is None else min(int(np.asarray(seqused)[s]), L)
        lo_i, hi_i = np.searchsorted(srows, [start, end])
        if hi_i <= lo_i:
            continue
        sel = order[lo_i:hi_i]  # output slots of rows in this sequence
        lq_all = rows[sel] - start
        keep = lq_all < u  # padded rows stay zero
        sel, lq_all = sel[keep], lq_all[keep]
        if len(sel) == 0:
            continue
        k_lo = 0 if window == 0 else max(0, int(lq_all.min()) - (window - 1))
        k_hi = int(lq_all.max()) + 1
        lk = np.arange(k_lo, k_hi, dtype=np.int64)
        kh = rms_norm(k[start + k_lo:start + k_hi], k_norm_w, eps)
        qh = rms_norm(q[start + lq_all], q_norm_w, eps)
        if use_rope:
            pk = lk if pos_all is None else pos_all[start + lk]
            pq = lq_all if pos_all is None else pos_all[start + lq_all]
            kh = rope_neox(kh, pk, theta)
            qh = rope_neox(qh, pq, theta)
        vv = v[start + k_lo:start + k_hi]
        nb = _row_block_size(len(lk), H)
        for b0 in range(0, len(sel), nb):
            bsel = sel[b0:b0 + nb]
            blq = lq_all[b0:b0 + nb]
            A = allowed_keys(blq, lk, u, window)  # [nb, nk]
            for h in range(H):
                g = kv_head_of(h, H, G)
                z = (qh[b0:b0 + nb, h, :] @ kh[:, g, :].T) / math.sqrt(D)  # [nb, nk]
                z = np.where(A, z, -np.inf)
                w_, ps, m, E = sink_softmax(z, sinks[h])
                out[bsel, h, :] = w_ @ vv[:, g, :]
                if dbg is not None:
                    dbg["weights"][bsel[:, None], h, lk[None, :]] = w_
                    dbg["p_sink"][bsel, h] = ps
                    dbg["m"][bsel, h] = m
                    dbg["E"][bsel, h] = E
    if debug:
        return out, dbg
    return out
