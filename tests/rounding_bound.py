"""First-order output error of the bf16 roundings in the attention kernel.

Used to grade cases where the plain bf16 bar is ill-conditioned (large RMSNorm
weights, near one-hot rows): the kernel rounds q', k' and P to bf16 once each,
and the resulting logit and weight perturbations move the output by an amount
computed here, row by row, from the oracle's own softmax weights.
"""

import numpy as np

from oracle import rms_norm, rope_neox

from .common import f64, i64, oracle_for

U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits, round to nearest even)


def perturbation_sigma(wl, layer, rows):
    """Per-element standard deviation of the output error that the single bf16
    rounding of q', k' and P leaves, to first order.

    The kernel multiplies q' = bf16(qhat log2(e) / sqrt(128)) and
    k' = bf16(khat), each element carrying an independent relative error e
    with |e| <= u = 2^-8, modelled as uniform (variance u^2 / 3). A logit
    z_i = qhat.khat_i / sqrt(128) then moves by
    dz_i = sum_c qhat_c khat_ic (e^q_c + e^k_ic) / sqrt(128), and the output of
    a row with softmax weights w_i moves by dO = sum_i w_i dz_i (v_i - O).
    The query errors are shared by all keys of the row, the key errors are
    not, so
      Var(dO_d) = u^2/3/128 [sum_c qhat_c^2 (sum_i w_i khat_ic (v_id - O_d))^2
                              + sum_i w_i^2 (v_id - O_d)^2 sum_c qhat_c^2 khat_ic^2]
    plus the rounding of P to bf16 (relative error per weight, the same values
    in numerator and denominator): u^2/3 sum_i w_i^2 (v_id - O_d)^2.
    Returns (sigma [rows, 32, 128], O [rows, 32, 128])."""
    q, k, v = f64(wl.q), f64(wl.k), f64(wl.v)
    qw, kw = f64(wl.q_norm_w), f64(wl.k_norm_w)
    cu = i64(wl.cu_seqlens)
    pos = i64(wl.positions)
    out, dbg = oracle_for(wl, layer, rows=rows, debug=True)
    W = dbg["weights"]  # [rows, 32, Lmax] by key index in the sequence
    sig = np.zeros_like(out)
    su = None if wl.seqused is None else i64(wl.seqused)
    for r_i, t in enumerate(rows):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        a, b = int(cu[s]), int(cu[s + 1])
        lq = t - a
        if su is not None and lq >= su[s]:
            continue  # a padded row is exactly zero
        lo = 0 if layer.window == 0 else max(0, lq - layer.window + 1)
        keys = np.arange(lo, lq + 1)
        kh = rms_norm(k[a + keys], kw, layer.eps)
        qh = rms_norm(q[t:t + 1], qw, layer.eps)
        if layer.use_rope:
            pk = keys if pos is None else pos[a + keys]
            pq = np.array([lq]) if pos is None else pos[t:t + 1]
            kh = rope_neox(kh, pk, layer.theta)
            qh = rope_neox(qh, pq, layer.theta)
        for h in range(32):
            g = h // 8
            w = W[r_i, h, keys]                       # [n]
            dv = v[a + keys, g, :] - out[r_i, h][None, :]   # [n, 128]
            kg = kh[:, g, :]                           # [n, 128]
            qc2 = qh[0, h, :] ** 2                     # [128]
            A = (kg * w[:, None]).T @ dv               # [128 c, 128 d]
            v1 = qc2 @ (A * A)                         # [128 d]
            v2 = ((w[:, None] * dv) ** 2 * ((kg * kg) @ qc2)[:, None]).sum(0)
            vp = ((w[:, None] * dv) ** 2).sum(0)
            var = U_BF16 ** 2 / 3.0 * ((v1 + v2) / 128.0 + vp)
            sig[r_i, h] = np.sqrt(var)
    return sig, out
