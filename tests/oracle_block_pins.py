"""Pins of the attention-block oracle (projections around the layer).

Each ``pin_*`` raises AssertionError when the oracle breaks the fact it checks
and looks the oracle up at call time, so a test can plant a mistake in it. The
facts (flint.layers page, ``FlintAttention``: separate q/k/v projections
without bias, then the layer, then ``o_proj``):

  - brute force: projections and the output projection by explicit loops over
    channels (W is [out, in]; channel h * head_dim + d is head h, channel d),
    with the layer itself from the separately pinned layer oracle;
  - permuting the query heads inside a kv group (their q rows, sinks and o_proj
    columns together) leaves the block's output unchanged;
  - the block is linear in the value and output weights;
  - padded tokens output zero.
"""

from __future__ import annotations

import numpy as np

import oracle.flint_oracle as fo
import oracle.flint_oracle_block as fb

HID, H, G, D = 12, 4, 2, 4


def _draw(seed, T):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (T, HID))
    w = dict(w_q=rng.normal(0, 0.3, (H * D, HID)), w_k=rng.normal(0, 0.3, (G * D, HID)),
             w_v=rng.normal(0, 0.3, (G * D, HID)), w_o=rng.normal(0, 0.3, (HID, H * D)))
    p = dict(q_norm_w=rng.normal(1, 0.2, D), k_norm_w=rng.normal(1, 0.2, D),
             sinks=rng.normal(0, 1, H))
    return x, w, p


def _block(x, w, p, cu, **kw):
    return fb.flint_attention_block(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], p["q_norm_w"],
                                    p["k_norm_w"], p["sinks"], cu, head_dim=D, theta=1e4, **kw)


def _close(a, b, what, tol=1e-12):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, f"{what}: max abs err {err:.3e}"


def pin_brute_force():
    T = 9
    x, w, p = _draw(1, T)
    cu = np.array([0, 5, 9])
    y, (q, k, v), o = _block(x, w, p, cu, window=3)
    qb = np.zeros((T, H, D))
    kb = np.zeros((T, G, D))
    vb = np.zeros((T, G, D))
    for t in range(T):
        for h in range(H):
            for d in range(D):
                qb[t, h, d] = sum(x[t, i] * w["w_q"][h * D + d, i] for i in range(HID))
        for g in range(G):
            for d in range(D):
                kb[t, g, d] = sum(x[t, i] * w["w_k"][g * D + d, i] for i in range(HID))
                vb[t, g, d] = sum(x[t, i] * w["w_v"][g * D + d, i] for i in range(HID))
    _close(q, qb, "q projection")
    _close(k, kb, "k projection")
    _close(v, vb, "v projection")
    ob = fo.flint_attention(qb, kb, vb, p["q_norm_w"], p["k_norm_w"], p["sinks"], cu, window=3,
                            theta=1e4)
    yb = np.zeros((T, HID))
    for t in range(T):
        for c in range(HID):
            yb[t, c] = sum(ob[t, h, d] * w["w_o"][c, h * D + d] for h in range(H) for d in range(D))
    _close(y, yb, "output projection")


def pin_head_permutation():
    T = 11
    x, w, p = _draw(2, T)
    cu = np.array([0, T])
    y, _, _ = _block(x, w, p, cu, window=0, use_rope=False)
    perm = np.array([1, 0, 3, 2])  # swaps heads inside each kv group of 2
    ch = (perm[:, None] * D + np.arange(D)[None, :]).reshape(-1)
    w2 = dict(w)
    w2["w_q"] = w["w_q"][ch]
    w2["w_o"] = w["w_o"][:, ch]
    p2 = dict(p)
    p2["sinks"] = p["sinks"][perm]
    y2, _, _ = _block(x, w2, p2, cu, window=0, use_rope=False)
    _close(y, y2, "query heads permuted within their kv groups")


def pin_linear_in_value_and_output_weights():
    T = 8
    x, w, p = _draw(3, T)
    cu = np.array([0, T])
    y, _, _ = _block(x, w, p, cu, window=4)
    for name in ("w_v", "w_o"):
        w2 = dict(w)
        w2[name] = 2.5 * w[name]
        y2, _, _ = _block(x, w2, p, cu, window=4)
        _close(y2, 2.5 * y, f"linear in {name}")


def pin_padding_outputs_zero():
    T = 10
    x, w, p = _draw(4, T)
    cu = np.array([0, 6, 10])
    y, _, _ = _block(x, w, p, cu, seqused=np.array([4, 0]), window=0)
    assert np.all(y[4:6] == 0) and np.all(y[6:] == 0) and np.all(np.abs(y[:4]).sum(-1) > 0)


ALL_PINS = [
    pin_padding_outputs_zero,
    pin_linear_in_value_and_output_weights,
    pin_head_permutation,
    pin_brute_force,
]
