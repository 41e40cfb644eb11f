"""Pins of the FP64 oracle to facts other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle breaks the fact
it checks. The facts come from the pages (window of 513 that counts the current
token, zero-value unscaled sink, NeoX half rotation, norm before RoPE, padding
and document semantics), from library routines that compute the same thing a
different way (torch's ``rms_norm`` and ``scaled_dot_product_attention`` with
an extra key column for the sink, the GPT-NeoX rotary helpers in transformers),
from closed forms, and from scalar brute force on tiny inputs.

The functions look the oracle up at call time (``fo.flint_attention`` and
friends), so a test can plant a mistake in the oracle and check that some pin
catches it.
"""

from __future__ import annotations

import cmath
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle.flint_oracle as fo
from workload import Layer, make_custom
from workload.gen import FULL, SLIDING

from .common import f64, i64, oracle_for, seq_index

H, G, D = 32, 4, 128


# ---------------------------------------------------------------- references


def _torch_rms(x: torch.Tensor, w: torch.Tensor, eps: float) -> torch.Tensor:
    return F.rms_norm(x, (x.shape[-1],), weight=w, eps=eps)


def _neox_library_rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """NeoX rotation through transformers' GPT-NeoX ``apply_rotary_pos_emb``.

    x is [N, heads, D] float64. The inverse frequencies follow the library's
    default-RoPE expression, evaluated in float64 (the library evaluates the
    same expression in float32; ``pin_rope_frequencies_library`` ties the two).
    """
    from transformers.models.gpt_neox.modeling_gpt_neox import apply_rotary_pos_emb

    dim = x.shape[-1]
    inv = 1.0 / (theta ** (torch.arange(0, dim, 2, dtype=torch.float64) / dim))
    freqs = pos.to(torch.float64)[:, None] * inv[None, :]
    emb = torch.cat([freqs, freqs], dim=-1)  # [N, D]
    cos, sin = emb.cos(), emb.sin()
    xq = x.transpose(0, 1)[None]  # [1, heads, N, D]
    out, _ = apply_rotary_pos_emb(xq, xq, cos[None], sin[None], unsqueeze_dim=1)
    return out[0].transpose(0, 1).contiguous()


def _library_layer(wl, layer, sinks=None):
    """Whole layer via torch SDPA with one extra zero key whose mask is the sink.

    Returns O [T, H, D] float64 (padded rows zero).
    """
    q = wl.q.to(torch.float64)
    k = wl.k.to(torch.float64)
    v = wl.v.to(torch.float64)
    qw = wl.q_norm_w.to(torch.float64)
    kw = wl.k_norm_w.to(torch.float64)
    sk = (wl.sinks if sinks is None else torch.as_tensor(sinks)).to(torch.float64)
    T = q.shape[0]
    cu = i64(wl.cu_seqlens)
    out = torch.zeros(T, H, D, dtype=torch.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        u = L if wl.seqused is None else min(int(wl.seqused[s]), L)
        if u == 0:
            continue
        qh = _torch_rms(q[a:a + u], qw, layer.eps)
        kh = _torch_rms(k[a:a + u], kw, layer.eps)
        if layer.use_rope:
            pos = torch.arange(u) if wl.positions is None else wl.positions[a:a + u].to(torch.int64)
            qh = _neox_library_rope(qh, pos, layer.theta)
            kh = _neox_library_rope(kh, pos, layer.theta)
        idx = torch.arange(u)
        ok = idx[None, :] <= idx[:, None]
        if layer.window > 0:
            ok &= (idx[:, None] - idx[None, :]) <= layer.window - 1
        mask = torch.zeros(H, u, u + 1, dtype=torch.float64)
        mask[:, :, :u] = torch.where(ok, 0.0, -math.inf)[None]
        mask[:, :, u] = sk[:, None]
        kx = torch.cat([kh, torch.zeros(1, G, D, dtype=torch.float64)], 0)
        vx = torch.cat([v[a:a + u], torch.zeros(1, G, D, dtype=torch.float64)], 0)
        o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kx.transpose(0, 1)[None],
                                           vx.transpose(0, 1)[None], attn_mask=mask[None],
                                           enable_gqa=True)
        out[a:a + u] = o[0].transpose(0, 1)
    return out


def _plain_softmax_layer(wl, layer):
    """Standard causal (windowed) softmax attention via torch SDPA, no sink."""
    q = wl.q.to(torch.float64)
    k = wl.k.to(torch.float64)
    v = wl.v.to(torch.float64)
    T = q.shape[0]
    cu = i64(wl.cu_seqlens)
    out = torch.zeros(T, H, D, dtype=torch.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        u = (b - a) if wl.seqused is None else min(int(wl.seqused[s]), b - a)
        if u == 0:
            continue
        qh = _torch_rms(q[a:a + u], wl.q_norm_w.double(), layer.eps)
        kh = _torch_rms(k[a:a + u], wl.k_norm_w.double(), layer.eps)
        if layer.use_rope:
            pos = torch.arange(u) if wl.positions is None else wl.positions[a:a + u].to(torch.int64)
            qh = _neox_library_rope(qh, pos, layer.theta)
            kh = _neox_library_rope(kh, pos, layer.theta)
        idx = torch.arange(u)
        ok = idx[None, :] <= idx[:, None]
        if layer.window > 0:
            ok &= (idx[:, None] - idx[None, :]) <= layer.window - 1
        o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kh.transpose(0, 1)[None],
                                           v[a:a + u].transpose(0, 1)[None], attn_mask=ok[None, None],
                                           enable_gqa=True)
        out[a:a + u] = o[0].transpose(0, 1)
    return out


def _brute_force(wl, layer):
    """Scalar loops over a tiny workload; sink softmax as an explicit category list."""
    q = wl.q.double().tolist()
    k = wl.k.double().tolist()
    v = wl.v.double().tolist()
    qw = wl.q_norm_w.double().tolist()
    kw = wl.k_norm_w.double().tolist()
    sinks = wl.sinks.double().tolist()
    cu = [int(x) for x in wl.cu_seqlens.tolist()]
    T = len(q)
    pos_list = None if wl.positions is None else [int(x) for x in wl.positions.tolist()]

    def norm(vec, w):
        ms = math.fsum(x * x for x in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + layer.eps)
        return [x * r * wc for x, wc in zip(vec, w)]

    def rotate(vec, p):
        half = len(vec) // 2
        outv = [0.0] * len(vec)
        for c in range(half):
            z = complex(vec[c], vec[c + half]) * cmath.exp(1j * p * layer.theta ** (-c / half))
            outv[c], outv[c + half] = z.real, z.imag
        return outv

    out = np.zeros((T, H, D))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        u = (b - a) if wl.seqused is None else min(int(wl.seqused[s]), b - a)
        kh = {}
        for j in range(u):
            for g in range(G):
                x = norm(k[a + j][g], kw)
                if layer.use_rope:
                    x = rotate(x, j if pos_list is None else pos_list[a + j])
                kh[j, g] = x
        for i in range(u):
            # keys: the current token and the (window - 1) before it, or all before it
            first = 0 if layer.window == 0 else max(0, i - (layer.window - 1))
            keys = list(range(first, i + 1))
            for h in range(H):
                g = h // (H // G)
                x = norm(q[a + i][h], qw)
                if layer.use_rope:
                    x = rotate(x, i if pos_list is None else pos_list[a + i])
                logits = [math.fsum(xa * xb for xa, xb in zip(x, kh[j, g])) / math.sqrt(D)
                          for j in keys]
                cats = [math.exp(sinks[h])] + [math.exp(z) for z in logits]
                den = math.fsum(cats)
                for d in range(D):
                    out[a + i, h, d] = math.fsum(cats[1 + n] * v[a + j][g][d]
                                                 for n, j in enumerate(keys)) / den
    return out


def _close(a, b, rtol, atol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    lim = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert err <= lim, f"{what}: max abs err {err:.3e} > {lim:.3e}"


# ---------------------------------------------------------------- pins


def pin_rmsnorm_library():
    """Oracle RMSNorm equals torch.nn.functional.rms_norm (weight form, eps inside)."""
    rng = np.random.default_rng(11)
    for scale in (1.0, 1e-3, 3e-4):
        x = rng.standard_normal((40, 5, D)) * scale
        w = 1.0 + 0.1 * rng.standard_normal(D)
        ref = _torch_rms(torch.from_numpy(x), torch.from_numpy(w), 1e-6).numpy()
        _close(fo.rms_norm(x, w, 1e-6), ref, 1e-13, 0.0, f"rms_norm scale {scale}")


def pin_rmsnorm_closed_form():
    """With w = 1, mean(xhat^2) = ms / (ms + eps); with x -> c x only eps matters."""
    rng = np.random.default_rng(12)
    eps = 1e-6
    for scale in (1.0, 1e-3):
        x = rng.standard_normal((30, D)) * scale
        y = fo.rms_norm(x, np.ones(D), eps)
        ms = np.mean(x * x, axis=-1)
        _close(np.mean(y * y, axis=-1), ms / (ms + eps), 1e-13, 0.0, "mean(xhat^2)")
    x = rng.standard_normal((30, D))
    _close(fo.rms_norm(7.0 * x, np.ones(D), 0.0), fo.rms_norm(x, np.ones(D), 0.0), 1e-13, 0.0,
           "scale invariance at eps=0")


def pin_rope_frequencies_library():
    """Oracle RoPE frequencies equal the default-RoPE inverse frequencies of transformers."""
    from transformers import GPTNeoXConfig
    from transformers.models.gpt_neox.modeling_gpt_neox import GPTNeoXRotaryEmbedding

    for theta in (1.0e6, 1.0e4):
        cfg = GPTNeoXConfig(hidden_size=H * D, num_attention_heads=H, max_position_embeddings=262144,
                            rope_parameters={"rope_type": "default", "rope_theta": theta,
                                             "partial_rotary_factor": 1.0})
        lib = GPTNeoXRotaryEmbedding.compute_default_rope_parameters(cfg)[0].double().numpy()
        ours = fo.rope_frequencies(D, theta)
        _close(ours / lib, np.ones(D // 2), 1e-6, 0.0, f"inverse frequencies vs transformers, theta {theta}")


def pin_rope_library():
    """Oracle NeoX RoPE equals transformers' GPT-NeoX rotate-half rotation."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((50, 3, D))
    pos = rng.integers(0, 262144, 50)
    pos[:5] = [0, 1, 2, 512, 513]
    ref = _neox_library_rope(torch.from_numpy(x), torch.from_numpy(pos), 1.0e6).numpy()
    _close(fo.rope_neox(x, pos, 1.0e6), ref, 1e-9, 0.0, "rope vs GPT-NeoX apply_rotary_pos_emb")


def pin_rope_complex():
    """Channel c and c+64 form one complex number multiplied by exp(i p omega_c)."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((20, 2, D))
    pos = rng.integers(0, 10000, 20)
    y = fo.rope_neox(x, pos, 1.0e6)
    for n in range(20):
        for hh in range(2):
            for c in (0, 1, 17, 32, 63):
                z = complex(x[n, hh, c], x[n, hh, c + 64]) * cmath.exp(1j * pos[n] * 1.0e6 ** (-c / 64))
                assert abs(z.real - y[n, hh, c]) < 1e-9 and abs(z.imag - y[n, hh, c + 64]) < 1e-9, \
                    f"rope channel {c} at position {pos[n]}"


def pin_rope_invariants():
    """RoPE keeps norms, is the identity at position 0, and depends on relative positions only."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((30, 4, D))
    pos = rng.integers(0, 100000, 30)
    y = fo.rope_neox(x, pos, 1.0e6)
    _close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), 1e-13, 0.0, "rope norm")
    y0 = fo.rope_neox(x, np.zeros(30, np.int64), 1.0e6)
    assert np.array_equal(y0, x), "rope at position 0 must be the identity"
    a = rng.standard_normal((1, 1, D))
    b = rng.standard_normal((1, 1, D))
    dots = []
    for shift in (0, 5, 1000, 77777):
        ra = fo.rope_neox(a, np.array([300 + shift]), 1.0e6)
        rb = fo.rope_neox(b, np.array([100 + shift]), 1.0e6)
        dots.append(float(np.sum(ra * rb)))
    _close(np.array(dots), np.full(4, dots[0]), 1e-12, 1e-12, "relative-position invariance")


def _small_cases():
    return [
        (make_custom(101, [12], layers=[Layer(window=5, use_rope=True)]), Layer(window=5, use_rope=True)),
        (make_custom(102, [9], layers=[FULL]), FULL),
        (make_custom(103, [7, 5], layout="thd", layers=[Layer(window=3, use_rope=True)]),
         Layer(window=3, use_rope=True)),
        (make_custom(104, [10, 10], layout="bshd", seqused=[7, 10], positions="none"),
         Layer(window=4, use_rope=True)),
        (make_custom(105, [6], sink_std=4.0, positions="random"), Layer(window=2, use_rope=True)),
        (make_custom(106, [8], layers=[Layer(window=1, use_rope=False)]), Layer(window=1, use_rope=False)),
    ]


def pin_brute_force():
    """Scalar brute force on tiny inputs (all 32 heads) matches to 1e-12."""
    for wl, layer in _small_cases():
        ref = _brute_force(wl, layer)
        got = oracle_for(wl, layer)
        _close(got, ref, 1e-12, 1e-13, f"brute force seed {wl.seed}")


def pin_library_layer():
    """Whole layer equals torch SDPA (FP64) with a zero key whose additive mask is the sink."""
    cases = _small_cases() + [
        (make_custom(110, [700], layers=[SLIDING]), SLIDING),
        (make_custom(111, [300, 1, 650, 64], layout="thd"), SLIDING),
        (make_custom(112, [200, 170], layout="thd", positions="none"), FULL),
        (make_custom(113, [96, 96, 96], layout="bshd", seqused=[96, 40, 0]), FULL),
    ]
    for wl, layer in cases:
        ref = _library_layer(wl, layer).numpy()
        got = oracle_for(wl, layer)
        # positions up to 2^18 make FP64 angle rounding differ by ~1e-11 rad
        _close(got, ref, 1e-10, 1e-13, f"SDPA identity seed {wl.seed}")


def pin_sink_minus_inf_is_softmax():
    """A sink of -inf reduces the layer to standard softmax attention."""
    for wl, layer in [(make_custom(120, [70], layers=[SLIDING]), Layer(window=9, use_rope=True)),
                      (make_custom(121, [50, 30], layout="thd"), FULL)]:
        ref = _plain_softmax_layer(wl, layer).numpy()
        got = oracle_for(wl, layer, sinks=np.full(H, -np.inf))
        _close(got, ref, 1e-12, 1e-13, "sink=-inf vs plain softmax")


def pin_sink_plus_large():
    """A very large sink takes all the weight: O -> 0 and p_sink -> 1."""
    wl = make_custom(122, [40])
    o, dbg = oracle_for(wl, SLIDING, sinks=np.full(H, 700.0), debug=True)
    assert np.max(np.abs(o)) < 1e-250, "large sink must drive the output to zero"
    _close(dbg["p_sink"], np.ones_like(dbg["p_sink"]), 1e-15, 0.0, "p_sink -> 1")


def pin_weights_sum():
    """Row weights over the keys sum to exactly 1 - p_sink."""
    for wl, layer in [(make_custom(130, [600], sink_std=3.0), SLIDING),
                      (make_custom(131, [90, 50], layout="thd"), FULL)]:
        _, dbg = oracle_for(wl, layer, debug=True)
        tot = dbg["weights"].sum(-1) + dbg["p_sink"]
        _close(tot, np.ones_like(tot), 1e-14, 1e-14, "sum of weights + p_sink")
        assert np.all(dbg["p_sink"] > 0), "a finite sink always keeps some weight"


def pin_window_count():
    """|A(t)| = min(l+1, 513) on sliding layers, l+1 on full layers, with q = 0.

    With q = 0 every allowed key has weight exactly 1/(e^sink + |A|) > 0, so the
    count of positive weights is the size of the key set.
    """
    wl = make_custom(140, [1100], q_scale=0.0)
    for layer, expect in ((SLIDING, lambda l: np.minimum(l + 1, 513)), (FULL, lambda l: l + 1)):
        _, dbg = oracle_for(wl, layer, debug=True)
        counts = (dbg["weights"][:, 0, :] > 0).sum(-1)
        ell = np.arange(1100)
        assert np.array_equal(counts, expect(ell)), f"window count for {layer.name}"
    assert counts[600] == 601
    _, dbg = oracle_for(wl, SLIDING, debug=True)
    w = dbg["weights"][700, 5]
    assert w[700 - 512] > 0 and w[700 - 513] == 0, "window holds the current token and 512 before it"


def pin_closed_form_q0():
    """q = 0 gives O[t] = sum_A v / (e^sink + |A|), exactly."""
    for layer, seqused in ((SLIDING, None), (FULL, [60])):
        wl = make_custom(150, [90], layout="bshd", seqused=seqused, q_scale=0.0)
        got = oracle_for(wl, layer)
        v = f64(wl.v)
        s = f64(wl.sinks)
        u = 90 if seqused is None else seqused[0]
        ref = np.zeros_like(got)
        for t in range(u):
            lo = 0 if layer.window == 0 else max(0, t - layer.window + 1)
            vs = v[lo:t + 1].sum(0)  # [G, D]
            for h in range(H):
                ref[t, h] = vs[h // 8] / (math.exp(s[h]) + (t + 1 - lo))
        _close(got, ref, 1e-13, 1e-15, f"q=0 closed form {layer.name}")


def pin_nope_position_invariance():
    """Full (NoPE) layers ignore positions: output bitwise unchanged."""
    wl = make_custom(160, [80, 40], layout="thd", positions="local")
    a = oracle_for(wl, FULL)
    b = oracle_for(wl, FULL, positions=np.random.default_rng(1).integers(0, 262144, 120))
    assert np.array_equal(a, b), "NoPE output must not depend on positions"


def pin_rope_shift_invariance():
    """Shifting every position by the same amount leaves a RoPE layer's output unchanged."""
    wl = make_custom(161, [64], positions="local")
    a = oracle_for(wl, Layer(window=17, use_rope=True))
    b = oracle_for(wl, Layer(window=17, use_rope=True), positions=np.arange(64) + 12345)
    _close(b, a, 1e-11, 1e-12, "position shift")


def pin_thd_is_per_document():
    """Each packed document gives the same rows as a run on that document alone."""
    lengths = [33, 1, 70, 20]
    wl = make_custom(170, lengths, layout="thd")
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for layer in (Layer(window=25, use_rope=True), FULL):
        full = oracle_for(wl, layer)
        for d, n in enumerate(lengths):
            a, b = cu[d], cu[d + 1]
            alone = fo.flint_attention(f64(wl.q)[a:b], f64(wl.k)[a:b], f64(wl.v)[a:b],
                                       f64(wl.q_norm_w), f64(wl.k_norm_w), f64(wl.sinks), [0, n],
                                       positions=i64(wl.positions)[a:b], window=layer.window,
                                       use_rope=layer.use_rope)
            assert np.array_equal(full[a:b], alone), f"document {d} {layer.name}"


def pin_gqa_is_repeated_mha():
    """32 query heads over 4 KV heads equal 32 KV heads holding head h // 8's values."""
    wl = make_custom(171, [50, 30], layout="thd")
    for layer in (Layer(window=20, use_rope=True), FULL):
        a = oracle_for(wl, layer)
        rep = np.repeat(np.arange(G), H // G)
        b = oracle_for(wl, layer, k=f64(wl.k)[:, rep], v=f64(wl.v)[:, rep])
        _close(b, a, 1e-13, 1e-15, f"GQA vs MHA {layer.name}")


def pin_causality_and_window():
    """Later tokens and tokens outside the window never reach O[t]."""
    S = 80
    wl = make_custom(172, [S])
    layer = Layer(window=20, use_rope=True)
    base = oracle_for(wl, layer)
    t = 45
    k2, v2 = f64(wl.k).copy(), f64(wl.v).copy()
    k2[t + 1:] += 3.0
    v2[t + 1:] -= 5.0
    k2[:t - 19] *= -2.0  # indices <= t - window
    v2[:t - 19] += 9.0
    pert = oracle_for(wl, layer, k=k2, v=v2)
    assert np.array_equal(pert[t], base[t]), "keys after t or outside the window changed O[t]"
    v3 = f64(wl.v).copy()
    v3[t - 19] += 1.0  # the oldest key inside the window
    assert not np.allclose(oracle_for(wl, layer, v=v3)[t], base[t]), "oldest window key must count"


def pin_padding():
    """Garbage in padded slots leaves valid rows unchanged; padded rows are zero."""
    wl = make_custom(173, [40, 40, 40], layout="bshd", seqused=[25, 40, 1])
    for layer in (Layer(window=9, use_rope=True), FULL):
        base = oracle_for(wl, layer)
        q2, k2, v2 = f64(wl.q).copy(), f64(wl.k).copy(), f64(wl.v).copy()
        for a, u in ((0, 25), (80, 1)):
            q2[a + u:a + 40] = 1e6
            k2[a + u:a + 40] = -1e6
            v2[a + u:a + 40] = 1e9
        pert = oracle_for(wl, layer, q=q2, k=k2, v=v2)
        assert np.array_equal(pert, base), f"padding garbage leaked ({layer.name})"
        s, ell = seq_index(i64(wl.cu_seqlens), 120)
        pad = ell >= np.array([25, 40, 1])[s]
        assert np.all(base[pad] == 0.0), "padded rows must be exactly zero"


def pin_row_sampling():
    """Computing a subset of rows gives exactly those rows of the full output."""
    wl = make_custom(174, [150, 90], layout="thd")
    for layer in (SLIDING, FULL):
        full = oracle_for(wl, layer)
        rows = np.array([239, 0, 149, 150, 151, 77, 3])
        part = oracle_for(wl, layer, rows=rows)
        # BLAS may sum in another order for another row-block size
        _close(part, full[rows], 1e-14, 0.0, f"row sampling {layer.name}")


ALL_PINS = [
    pin_rmsnorm_library,
    pin_rmsnorm_closed_form,
    pin_rope_frequencies_library,
    pin_rope_library,
    pin_rope_complex,
    pin_rope_invariants,
    pin_brute_force,
    pin_library_layer,
    pin_sink_minus_inf_is_softmax,
    pin_sink_plus_large,
    pin_weights_sum,
    pin_window_count,
    pin_closed_form_q0,
    pin_nope_position_invariance,
    pin_rope_shift_invariance,
    pin_thd_is_per_document,
    pin_gqa_is_repeated_mha,
    pin_causality_and_window,
    pin_padding,
    pin_row_sampling,
]
