"""Pins of the FP64 backward oracle to facts other than the oracle itself.

As in ``oracle_pins``, each ``pin_*`` raises AssertionError when the oracle
breaks the fact it checks, and looks the oracle up at call time so a test can
plant a mistake and see a pin catch it. The facts:

  - central finite differences of the (separately pinned) forward oracle, for
    every input: q, k, v, both norm weights and the sinks, on tiny shapes with
    padding, documents, windows, RoPE at arbitrary positions;
  - torch autograd through a library formulation of the layer (torch's
    ``rms_norm``, RoPE as a complex rotation, ``scaled_dot_product_attention``
    with one extra zero key whose additive mask is the sink, K/V repeated per
    query head) at the real head shape (32 query heads, 4 kv heads, d = 128);
  - invariants: RMSNorm scale invariance (with eps = 0 the gradient of a head
    vector is orthogonal to it), the logit-scale identity <w_q, dw_q> =
    <w_k, dw_k> (scaling either weight scales every logit the same way), the
    value-sum identity (sum over keys of dv = sum over rows of (1 - p_sink) dO),
    a sink of -inf has zero adjoint;
  - a one-token closed form;
  - row and key sampling agree with the full computation.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle.flint_oracle as fo
import oracle.flint_oracle_bwd as fb
from workload import Layer, make_custom
from workload.gen import FULL, SLIDING, draw_dout

from .common import f64, i64, oracle_for

H, G, D = 32, 4, 128


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    lim = atol + rtol * (float(np.max(np.abs(b))) if b.size else 0.0)
    assert err <= lim, f"{what}: max abs err {err:.3e} > {lim:.3e}"


def _bwd(args, **over):
    a = dict(args)
    a.update(over)
    return fb.flint_attention_backward(**a)


def _wl_args(wl, layer, dout, **over):
    a = dict(q=f64(wl.q), k=f64(wl.k), v=f64(wl.v), q_norm_w=f64(wl.q_norm_w),
             k_norm_w=f64(wl.k_norm_w), sinks=f64(wl.sinks), cu_seqlens=i64(wl.cu_seqlens),
             dout=dout, seqused=i64(wl.seqused), positions=i64(wl.positions),
             window=layer.window, use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps)
    a.update(over)
    return a


# ---------------------------------------------------------------- finite differences


def _tiny_cases():
    """Tiny shapes (4 query heads over 2 kv heads, d = 8) covering the layer's cases."""
    rng = np.random.default_rng(2024)
    cases = []
    for name, lens, used, window, rope, pos, sink_scale in [
        ("window 3, rope, padding, random positions", [5, 4], [5, 3], 3, True, "random", 1.0),
        ("full causal, nope", [6], None, 0, False, None, 1.0),
        ("window 2, rope, three documents", [3, 1, 4], None, 2, True, "local", 2.0),
        ("full, rope, strong sinks", [5], None, 0, True, "local", 6.0),
    ]:
        T = sum(lens)
        Hq, Gk, Dd = 4, 2, 8
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        if pos == "random":
            positions = rng.integers(0, 50, size=T)
        elif pos == "local":
            positions = np.concatenate([np.arange(n) for n in lens])
        else:
            positions = None
        args = dict(q=rng.normal(size=(T, Hq, Dd)), k=rng.normal(size=(T, Gk, Dd)),
                    v=rng.normal(size=(T, Gk, Dd)), q_norm_w=rng.normal(1.0, 0.3, Dd),
                    k_norm_w=rng.normal(1.0, 0.3, Dd), sinks=rng.normal(0.0, sink_scale, Hq),
                    cu_seqlens=cu, dout=rng.normal(size=(T, Hq, Dd)),
                    seqused=None if used is None else np.array(used), positions=positions,
                    window=window, use_rope=rope, theta=100.0, eps=1e-6)
        cases.append((name, args))
    return cases


def _loss(args):
    """L = sum(dO * O) through the forward oracle."""
    fw = {k: v for k, v in args.items() if k != "dout"}
    o = fo.flint_attention(**fw)
    return float(np.sum(o * args["dout"]))


def _fd_grad(args, name, step=1e-5):
    x = np.array(args[name], np.float64)
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + step
        lp = _loss({**args, name: x})
        flat[i] = keep - step
        lm = _loss({**args, name: x})
        flat[i] = keep
        gf[i] = (lp - lm) / (2 * step)
    return g


def pin_finite_differences():
    """Every gradient equals central differences of the forward oracle's sum(dO * O)."""
    for what, args in _tiny_cases():
        got = _bwd(args)
        for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("q_norm_w", "dq_norm_w"),
                          ("k_norm_w", "dk_norm_w"), ("sinks", "dsink")]:
            ref = _fd_grad(args, name)
            # central differences with step 1e-5 are accurate to ~1e-9 here
            _close(got[key], ref, 2e-7, 1e-8, f"{what}: {key}")


# ---------------------------------------------------------------- library autograd


def _complex_rope(x, pos, theta):
    """NeoX RoPE as complex multiplication: (x_c + i x_{c+D/2}) e^{i pos omega_c}."""
    half = x.shape[-1] // 2
    om = theta ** (-torch.arange(half, dtype=torch.float64) * 2.0 / x.shape[-1])
    ang = pos.to(torch.float64)[:, None] * om[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def _library_grads(wl, layer, dout):
    q = wl.q.double().requires_grad_()
    k = wl.k.double().requires_grad_()
    v = wl.v.double().requires_grad_()
    qw = wl.q_norm_w.double().requires_grad_()
    kw = wl.k_norm_w.double().requires_grad_()
    sk = wl.sinks.double().requires_grad_()
    T = q.shape[0]
    cu = i64(wl.cu_seqlens)
    outs = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        u = (b - a) if wl.seqused is None else min(int(wl.seqused[s]), b - a)
        if u == 0:
            continue
        qh = F.rms_norm(q[a:a + u], (D,), weight=qw, eps=layer.eps)
        kh = F.rms_norm(k[a:a + u], (D,), weight=kw, eps=layer.eps)
        if layer.use_rope:
            pos = torch.arange(u) if wl.positions is None else wl.positions[a:a + u].to(torch.int64)
            qh = _complex_rope(qh, pos, layer.theta)
            kh = _complex_rope(kh, pos, layer.theta)
        idx = torch.arange(u)
        ok = idx[None, :] <= idx[:, None]
        if layer.window > 0:
            ok &= (idx[:, None] - idx[None, :]) <= layer.window - 1
        mask = torch.cat([torch.where(ok, 0.0, -math.inf)[None].expand(H, u, u).double(),
                          sk[:, None, None].expand(H, u, 1)], dim=-1)
        kx = torch.cat([kh, torch.zeros(1, G, D, dtype=torch.float64)], 0)
        vx = torch.cat([v[a:a + u], torch.zeros(1, G, D, dtype=torch.float64)], 0)
        kr = kx.repeat_interleave(H // G, dim=1)
        vr = vx.repeat_interleave(H // G, dim=1)
        o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kr.transpose(0, 1)[None],
                                           vr.transpose(0, 1)[None], attn_mask=mask[None])
        outs.append((a, u, o[0].transpose(0, 1)))
    loss = sum((o * torch.as_tensor(dout[a:a + u])).sum() for a, u, o in outs)
    loss.backward()
    return {"dq": q.grad.numpy(), "dk": k.grad.numpy(), "dv": v.grad.numpy(),
            "dq_norm_w": qw.grad.numpy(), "dk_norm_w": kw.grad.numpy(), "dsink": sk.grad.numpy()}


def _library_cases():
    return [
        (make_custom(501, [70, 33], layers=[SLIDING]), Layer(window=9, use_rope=True)),
        (make_custom(502, [40, 1, 25], positions="random"), Layer(window=513, use_rope=True,
                                                                 theta=1.0e4)),
        (make_custom(503, [48, 48], layout="bshd", seqused=[48, 20]), FULL),
        (make_custom(504, [60], sink_std=5.0), FULL),
    ]


def pin_library_autograd():
    """Gradients equal torch autograd through rms_norm, a complex rotation and SDPA (FP64)."""
    for wl, layer in _library_cases():
        dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
        ref = _library_grads(wl, layer, dout)
        got = _bwd(_wl_args(wl, layer, dout))
        for key in ref:
            _close(got[key], ref[key], 1e-10, 1e-13, f"seed {wl.seed}: {key}")


# ---------------------------------------------------------------- invariants


def pin_rmsnorm_scale_invariance():
    """With eps = 0, RMSNorm ignores the scale of a head vector: <x, dx> = 0 per token and head."""
    wl = make_custom(510, [50, 30], layers=[SLIDING])
    layer = Layer(window=9, use_rope=True, eps=0.0)
    dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
    got = _bwd(_wl_args(wl, layer, dout))
    for x, dx, what in [(f64(wl.q), got["dq"], "q"), (f64(wl.k), got["dk"], "k")]:
        dots = np.sum(x * dx, axis=-1)
        scale = np.max(np.abs(x)) * np.max(np.abs(dx))
        assert np.max(np.abs(dots)) <= 1e-12 * scale * D, f"<{what}, d{what}> not zero"


def pin_logit_scale_identity():
    """<w_q, dw_q> = <w_k, dw_k>: scaling either norm weight scales every logit alike."""
    for wl, layer in [(make_custom(511, [64, 17], layers=[SLIDING]), Layer(window=9, use_rope=True)),
                      (make_custom(512, [45]), FULL)]:
        dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
        got = _bwd(_wl_args(wl, layer, dout))
        a = float(np.dot(f64(wl.q_norm_w), got["dq_norm_w"]))
        b = float(np.dot(f64(wl.k_norm_w), got["dk_norm_w"]))
        assert abs(a - b) <= 1e-10 * max(abs(a), abs(b), 1e-30), f"{a} vs {b}"
        assert abs(a) > 1e-6, "identity checked on a non-trivial value"


def pin_value_sum_identity():
    """sum_j dv[j, g] = sum over rows t and heads h of group g of (1 - p_sink[t, h]) dO[t, h]."""
    wl = make_custom(513, [80, 24], layers=[SLIDING], sink_std=3.0)
    layer = Layer(window=9, use_rope=True)
    dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
    got = _bwd(_wl_args(wl, layer, dout))
    _, dbg = oracle_for(wl, layer, debug=True)
    w = (1.0 - dbg["p_sink"])[:, :, None] * dout  # [T, H, D]
    ref = w.reshape(-1, G, H // G, D).sum(axis=(0, 2))
    _close(got["dv"].sum(axis=0), ref, 1e-12, 1e-13, "value sum")


def pin_sink_minus_inf():
    """A sink of -inf has probability 0, so its adjoint is 0; other gradients stay finite."""
    wl = make_custom(514, [40])
    dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
    got = _bwd(_wl_args(wl, FULL, dout, sinks=np.full(H, -np.inf)))
    assert np.all(got["dsink"] == 0.0)
    for key in ("dq", "dk", "dv", "dq_norm_w", "dk_norm_w"):
        assert np.all(np.isfinite(got[key])), key


def pin_one_token_closed_form():
    """One token sees only itself: O = (1 - p) v with p = 1 / (1 + exp(z - sink)).

    Then dL/dv = (1 - p) dO, dL/dsink = -p (1 - p) dO.v and the logit z gets
    p (1 - p) dO.v, which makes dq' = that times k'/sqrt(D).
    """
    rng = np.random.default_rng(515)
    Hq, Gk, Dd = 2, 1, 4
    q = rng.normal(size=(1, Hq, Dd))
    k = rng.normal(size=(1, Gk, Dd))
    v = rng.normal(size=(1, Gk, Dd))
    do = rng.normal(size=(1, Hq, Dd))
    ones = np.ones(Dd)
    sinks = np.array([0.3, -1.2])
    got = fb.flint_attention_backward(q, k, v, ones, ones, sinks, [0, 1], do, window=513,
                                      use_rope=False, eps=0.0)
    qn = q[0] / np.sqrt(np.mean(q[0] ** 2, axis=-1, keepdims=True))
    kn = k[0, 0] / np.sqrt(np.mean(k[0, 0] ** 2))
    for h in range(Hq):
        z = float(qn[h] @ kn) / math.sqrt(Dd)
        p = 1.0 / (1.0 + math.exp(z - sinks[h]))
        dov = float(do[0, h] @ v[0, 0])
        assert abs(got["dsink"][h] - (-p * (1 - p) * dov)) <= 1e-14, h
        # dq' = p(1-p) dO.v k'/sqrt(D); through the norm (eps = 0, w = 1):
        # dq = r (dq' - qn mean(qn dq'))
        dqp = p * (1 - p) * dov * kn / math.sqrt(Dd)
        r = 1.0 / math.sqrt(float(np.mean(q[0, h] ** 2)))
        dq = r * (dqp - qn[h] * np.mean(qn[h] * dqp))
        _close(got["dq"][0, h], dq, 1e-13, 1e-15, f"dq head {h}")
    dv = sum((1 - 1.0 / (1.0 + math.exp(float(qn[h] @ kn) / math.sqrt(Dd) - sinks[h]))) * do[0, h]
             for h in range(Hq))
    _close(got["dv"][0, 0], dv, 1e-14, 1e-15, "dv")


def pin_forward_by_products():
    """out equals the forward oracle, and lse = m + log E of its softmax."""
    wl = make_custom(516, [70, 20], layers=[SLIDING], seqused=None)
    layer = Layer(window=9, use_rope=True)
    dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
    got = _bwd(_wl_args(wl, layer, dout))
    o, dbg = oracle_for(wl, layer, debug=True)
    _close(got["out"], o, 1e-14, 0.0, "out")
    _close(got["lse"], dbg["m"] + np.log(dbg["E"]), 1e-14, 0.0, "lse")


def pin_sampling():
    """Gradients of selected rows / keys equal the full computation's."""
    wl = make_custom(517, [150, 90], layers=[SLIDING], seqused=None)
    for layer in (Layer(window=9, use_rope=True), FULL):
        dout = f64(draw_dout(wl.seed, wl.q.shape[0]))
        args = _wl_args(wl, layer, dout)
        full = _bwd(args)
        rows = np.array([239, 0, 149, 150, 151, 77, 3])
        keys = np.array([5, 149, 150, 200, 0, 239])
        part = _bwd(args, rows=rows, keys=keys)
        _close(part["dq"], full["dq"][rows], 1e-13, 0.0, "dq rows")
        _close(part["dk"], full["dk"][keys], 1e-13, 0.0, "dk keys")
        _close(part["dv"], full["dv"][keys], 1e-13, 0.0, "dv keys")
        _close(part["dsink"], full["dsink"], 1e-13, 0.0, "dsink")
        assert part["dq_norm_w"] is None and part["dk_norm_w"] is None


ALL_PINS = [
    pin_one_token_closed_form,
    pin_sink_minus_inf,
    pin_forward_by_products,
    pin_value_sum_identity,
    pin_logit_scale_identity,
    pin_rmsnorm_scale_invariance,
    pin_sampling,
    pin_library_autograd,
    pin_finite_differences,
]
