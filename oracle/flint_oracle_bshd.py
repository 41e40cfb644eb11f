"""FP64 CPU oracle of the Flint sink attention on BSHD input with document ids
and arbitrary padding.

TEST INFRASTRUCTURE ONLY, like the other oracle modules: only the tests, the
package's ``smoke()`` check and the CPU-baseline leg of the benchmark may import
it; the product path never does, and nothing is shared with it.

The flint.layers API page (``FlintAttention.forward``, its ``attention_mask``
and ``attn_kwargs`` arguments) describes the inputs:
  * ``attention_mask`` [B, S], one for a valid token. Padded queries and keys
    leave real attention; the zero-value sink stays valid. Trailing padding is
    what TE's BSHD path takes; arbitrary padding is handled by THD packing, so
    the layer behaves as the THD layer on the row's valid tokens in order.
  * ``document_ids`` [B, S] integers for a block-diagonal mask: a query sees
    only keys of its own document.
  * positions [B, S] optional; by default contiguous zero-based positions,
    which for packed documents means the index inside the document.

This module writes that definition out per row, one dense [S, S] mask at a
time, with these readings of what the pages leave open:
  * documents are the maximal runs of equal id among the row's valid tokens
    (the blocks of a block-diagonal mask); an id that comes back after another
    id starts a new document;
  * the window counts valid tokens of the document (the packed order), not
    columns of the row, as THD packing does: the key is allowed when at most
    window-1 valid tokens of the document separate it from the query;
  * default positions are the index among the document's valid tokens (RoPE
    logits depend on position differences only, so any per-document shift
    gives the same exact result; counting row columns would not, where a
    document has holes).
Every other step (RMSNorm, NeoX RoPE, logit scale, sink softmax, GQA) is the
forward oracle's, with the same page citations.
"""

from __future__ import annotations

import math

import numpy as np

from . import flint_oracle as fo

__all__ = ["document_structure", "flint_attention_bshd"]


def document_structure(valid: np.ndarray, doc_ids: np.ndarray):
    """For one row: (rank, doc, local) per column.

    rank  = index among the row's valid tokens (-1 on padding),
    doc   = document number: a new one starts at the first valid token and at
            every valid token whose id differs from the previous valid token's
            (-1 on padding),
    local = index of the token inside its document (-1 on padding).
    """
    S = len(valid)
    rank = np.full(S, -1, np.int64)
    doc = np.full(S, -1, np.int64)
    local = np.full(S, -1, np.int64)
    r = 0
    d = -1
    prev_id = None
    start_rank = 0
    for s in range(S):
        if not valid[s]:
            continue
        if prev_id is None or doc_ids[s] != prev_id:
            d += 1
            start_rank = r
        rank[s] = r
        doc[s] = d
        local[s] = r - start_rank
        prev_id = doc_ids[s]
        r += 1
    return rank, doc, local


def _allowed(rank, doc, window: int) -> np.ndarray:
    """Boolean [S, S]: key column j is allowed for query column t."""
    rq, rk = rank[:, None], rank[None, :]
    ok = (rq >= 0) & (rk >= 0) & (doc[:, None] == doc[None, :]) & (rk <= rq)
    if window > 0:
        ok &= (rq - rk) <= (window - 1)
    return ok


def flint_attention_bshd(q, k, v, q_norm_w, k_norm_w, sinks, attention_mask=None,
                         document_ids=None, position_ids=None, window: int = 513,
                         use_rope: bool = True, theta: float = 1.0e6,
                         eps: float = 1.0e-6) -> np.ndarray:
    """Sink-aware GQA forward in FP64 on q [B, S, H, D], k and v [B, S, G, D].

    attention_mask, document_ids, position_ids: [B, S] or None. Returns
    out [B, S, H, D]; padded tokens output exactly zero.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sinks = np.asarray(sinks, np.float64)
    B, S, H, D = q.shape
    G = k.shape[2]
    out = np.zeros((B, S, H, D))
    for b in range(B):
        valid = np.ones(S, bool) if attention_mask is None else np.asarray(attention_mask[b]) != 0
        ids = np.zeros(S, np.int64) if document_ids is None else np.asarray(document_ids[b], np.int64)
        rank, doc, local = document_structure(valid, ids)
        pos = local if position_ids is None else np.asarray(position_ids[b], np.int64)
        qh = fo.rms_norm(q[b], q_norm_w, eps)
        kh = fo.rms_norm(k[b], k_norm_w, eps)
        if use_rope:
            qh = fo.rope_neox(qh, pos, theta)
            kh = fo.rope_neox(kh, pos, theta)
        A = _allowed(rank, doc, window)
        rows = np.nonzero(valid)[0]
        for h in range(H):
            g = fo.kv_head_of(h, H, G)
            z = np.where(A[rows], (qh[rows, h, :] @ kh[:, g, :].T) / math.sqrt(D), -np.inf)
            W, _, _, _ = fo.sink_softmax(z, sinks[h])
            out[b, rows, h, :] = W @ v[b, :, g, :]
    return out
