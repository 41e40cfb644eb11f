"""Pins of the BSHD document/padding oracle to facts other than itself.

Each ``pin_*`` raises AssertionError when the oracle breaks the fact it checks
and looks the oracle up at call time, so a test can plant a mistake in it and
see a pin catch it. The facts (flint.layers page, ``FlintAttention.forward``:
padded queries and keys leave attention, arbitrary padding is THD packing,
document ids give a block-diagonal mask):

  - trailing padding is the THD layer with per-sequence valid lengths;
  - documents without padding are THD sequences with boundaries at the runs;
  - interior holes: the row's valid tokens, packed in order and cut at the
    document runs, are THD sequences (with and without explicit positions);
  - values at padded tokens change nothing, and padded rows are exact zeros;
  - documents are runs: renaming ids changes nothing, an id that returns after
    another starts a new document;
  - brute force: every output of a tiny case by explicit loops over keys;
  - one-token documents have a closed form.
The THD oracle these compare with is pinned on its own (``oracle_pins``).
"""

from __future__ import annotations

import math

import numpy as np

import oracle.flint_oracle as fo
import oracle.flint_oracle_bshd as fd

H, G, D = 4, 2, 16
THETA = 1.0e4


def _draw(seed, B, S):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, (B, S, H, D))
    k = rng.normal(0, 1, (B, S, G, D))
    v = rng.normal(0, 1, (B, S, G, D))
    qw = rng.normal(1, 0.3, D)
    kw = rng.normal(1, 0.3, D)
    sk = rng.normal(0, 1, H)
    return q, k, v, qw, kw, sk


def _close(a, b, what, tol=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e}"


def _thd(q, k, v, qw, kw, sk, lengths, window, rope, positions=None, seqused=None):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return fo.flint_attention(q, k, v, qw, kw, sk, cu, seqused=seqused, positions=positions,
                              window=window, use_rope=rope, theta=THETA)


def _runs(lengths):
    """Document ids for consecutive runs of the given lengths (ids 10, 11, ...)."""
    return np.concatenate([np.full(n, 10 + i, np.int64) for i, n in enumerate(lengths)])


def pin_trailing_padding_is_thd():
    B, S = 3, 40
    q, k, v, qw, kw, sk = _draw(1, B, S)
    used = [40, 17, 0]
    mask = np.zeros((B, S), np.int64)
    for b, u in enumerate(used):
        mask[b, :u] = 1
    for window, rope in ((5, True), (0, False)):
        got = fd.flint_attention_bshd(q, k, v, qw, kw, sk, attention_mask=mask, window=window,
                                      use_rope=rope, theta=THETA)
        ref = _thd(q.reshape(B * S, H, D), k.reshape(B * S, G, D), v.reshape(B * S, G, D), qw, kw,
                   sk, [S] * B, window, rope, seqused=np.array(used))
        _close(got.reshape(B * S, H, D), ref, f"trailing padding w={window}")


def pin_documents_are_thd_sequences():
    B, S = 2, 50
    q, k, v, qw, kw, sk = _draw(2, B, S)
    lens = [[12, 1, 20, 17], [50]]
    ids = np.stack([_runs(x) for x in lens])
    for window, rope in ((7, True), (0, True), (0, False)):
        got = fd.flint_attention_bshd(q, k, v, qw, kw, sk, document_ids=ids, window=window,
                                      use_rope=rope, theta=THETA)
        ref = _thd(q.reshape(B * S, H, D), k.reshape(B * S, G, D), v.reshape(B * S, G, D), qw, kw,
                   sk, lens[0] + lens[1], window, rope)
        _close(got.reshape(B * S, H, D), ref, f"documents w={window} rope={rope}")


def pin_holes_pack_like_thd():
    B, S = 2, 40
    q, k, v, qw, kw, sk = _draw(3, B, S)
    rng = np.random.default_rng(33)
    mask = (rng.random((B, S)) > 0.3).astype(np.int64)
    mask[:, 0] = 0  # leading padding
    ids = np.stack([_runs([15, 25]), _runs([3, 30, 7])])
    pos_ids = rng.integers(0, 5000, (B, S))
    for window, explicit in ((4, False), (4, True), (0, False)):
        got = fd.flint_attention_bshd(q, k, v, qw, kw, sk, attention_mask=mask, document_ids=ids,
                                      position_ids=pos_ids if explicit else None, window=window,
                                      use_rope=True, theta=THETA)
        # pack by hand: the valid tokens of each row in order, cut where the id changes
        sel = [(b, s) for b in range(B) for s in range(S) if mask[b, s]]
        lengths = []
        for i, (b, s) in enumerate(sel):
            new = i == 0 or sel[i - 1][0] != b or ids[sel[i - 1]] != ids[b, s]
            if new:
                lengths.append(0)
            lengths[-1] += 1
        bi = np.array([x[0] for x in sel])
        si = np.array([x[1] for x in sel])
        ref = _thd(q[bi, si], k[bi, si], v[bi, si], qw, kw, sk, lengths, window, True,
                   positions=pos_ids[bi, si] if explicit else None)
        _close(got[bi, si], ref, f"holes w={window} explicit positions={explicit}")
        assert np.all(got[mask == 0] == 0.0)


def pin_padding_values_do_not_matter():
    B, S = 2, 30
    q, k, v, qw, kw, sk = _draw(4, B, S)
    rng = np.random.default_rng(44)
    mask = (rng.random((B, S)) > 0.4).astype(np.int64)
    ids = np.stack([_runs([10, 20]), _runs([30])])
    a = fd.flint_attention_bshd(q, k, v, qw, kw, sk, attention_mask=mask, document_ids=ids,
                                window=6, theta=THETA)
    pad = mask == 0
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[pad] = rng.normal(0, 50, q2[pad].shape)
    k2[pad] = rng.normal(0, 50, k2[pad].shape)
    v2[pad] = rng.normal(0, 50, v2[pad].shape)
    b = fd.flint_attention_bshd(q2, k2, v2, qw, kw, sk, attention_mask=mask, document_ids=ids,
                                window=6, theta=THETA)
    assert np.array_equal(a, b), "padded values leak into the output"
    assert np.all(a[pad] == 0.0) and np.all(np.abs(a[~pad]).sum(-1) > 0)


def pin_documents_are_runs():
    B, S = 1, 24
    q, k, v, qw, kw, sk = _draw(5, B, S)
    ids_a = np.array([[0] * 8 + [1] * 6 + [0] * 10])
    ids_b = np.array([[5] * 8 + [7] * 6 + [9] * 10])
    a = fd.flint_attention_bshd(q, k, v, qw, kw, sk, document_ids=ids_a, window=0, theta=THETA)
    b = fd.flint_attention_bshd(q, k, v, qw, kw, sk, document_ids=ids_b, window=0, theta=THETA)
    _close(a, b, "renamed ids", tol=0.0)
    alone = fd.flint_attention_bshd(q[:, 14:], k[:, 14:], v[:, 14:], qw, kw, sk, window=0,
                                    theta=THETA)
    _close(a[:, 14:], alone, "the returning id is a new document")


def pin_brute_force():
    """Each output by loops: walk the row, count the document's valid tokens
    between key and query, exponentiate logit by logit."""
    B, S, W = 1, 14, 3
    q, k, v, qw, kw, sk = _draw(6, B, S)
    mask = np.array([[0, 1, 1, 0, 1, 1, 1, 0, 0, 1, 1, 1, 1, 0]])
    ids = np.array([[4, 4, 4, 4, 4, 8, 8, 8, 8, 8, 2, 2, 2, 2]])
    got = fd.flint_attention_bshd(q, k, v, qw, kw, sk, attention_mask=mask, document_ids=ids,
                                  window=W, use_rope=True, theta=THETA)
    qn = fo.rms_norm(q[0], qw, 1e-6)
    kn = fo.rms_norm(k[0], kw, 1e-6)
    for t in range(S):
        if not mask[0, t]:
            assert np.all(got[0, t] == 0)
            continue
        # this token's document: valid tokens back to the last id change
        doc = [t]
        j = t - 1
        while j >= 0:
            if mask[0, j]:
                if ids[0, j] != ids[0, t]:
                    break
                doc.insert(0, j)
            j -= 1
        pos_t = len(doc) - 1
        qt = fo.rope_neox(qn[t][None], np.array([pos_t]), THETA)[0]
        for h in range(H):
            g = h // (H // G)
            num = np.zeros(D)
            den = math.exp(sk[h])
            for i, j in enumerate(doc):
                if pos_t - i > W - 1:
                    continue
                kj = fo.rope_neox(kn[j][None], np.array([i]), THETA)[0]
                e = math.exp(float(np.dot(qt[h], kj[g])) / math.sqrt(D))
                num += e * v[0, j, g]
                den += e
            _close(got[0, t, h], num / den, f"brute force t={t} h={h}", tol=1e-12)


def pin_one_token_documents():
    B, S = 1, 9
    q, k, v, qw, kw, sk = _draw(7, B, S)
    ids = np.arange(S)[None]
    got = fd.flint_attention_bshd(q, k, v, qw, kw, sk, document_ids=ids, window=0, use_rope=True,
                                  theta=THETA)
    qn = fo.rms_norm(q[0], qw, 1e-6)  # position 0 everywhere: RoPE is the identity
    kn = fo.rms_norm(k[0], kw, 1e-6)
    for t in range(S):
        for h in range(H):
            g = h // (H // G)
            z = float(np.dot(qn[t, h], kn[t, g])) / math.sqrt(D)
            p = 1.0 / (1.0 + math.exp(sk[h] - z))
            _close(got[0, t, h], p * v[0, t, g], f"one-token document t={t} h={h}", tol=1e-12)


ALL_PINS = [
    pin_one_token_documents,
    pin_documents_are_runs,
    pin_padding_values_do_not_matter,
    pin_trailing_padding_is_thd,
    pin_documents_are_thd_sequences,
    pin_holes_pack_like_thd,
    pin_brute_force,
]
