"""GPU parity of the backward (and the forward's row normalizer) against the FP64 oracle.

Tolerance, per gradient tensor X against the oracle's X_ref over valid tokens:
max |X - X_ref| <= 2e-2 * max |X_ref| and ||X - X_ref||_2 <= 1e-2 * ||X_ref||_2.
The HIP path multiplies bf16 operands (Q', K', V, dO, and the recomputed
softmax weights and logit gradients, each rounded once, relative error 2^-9)
with FP32 accumulation and rounds dq, dk, dv to bf16 once more; with random
rounding signs that gives a relative RMS error of a few 2^-9 = 2e-3, which
the bar leaves a factor of ~2.5 above. The parameter gradients (FP32 sums of
terms built from the same operands) take |err| <= 1e-2 * sum |terms|, where
the term scale is bounded by the oracle's sum of |X_ref| over the same
entries times 4 (a generous bound: individual terms cancel). Padded tokens
get exact zero gradients. The row normalizer lse: |err| <= 2e-2 + 4e-3 |lse|.
Its largest logits dominate it, and a logit made from bf16 operands (q' with
the softmax scale, k', each rounded once) carries a relative error of a few
2^-9, so the error grows with the logits' size (|lse| tracks the largest
logit); the denominator adds the bf16 rounding of the weights it sums,
2^-9 relative, i.e. about 2e-3 absolute.
"""

from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import flint_attention_backward
from workload import Layer, make_custom, make_workload
from workload.gen import FULL, SLIDING, draw_dout

from .common import f64, i64
from .gpu_common import huge_positions, to_np, valid_rows

pytestmark = pytest.mark.gpu

MAX_FRAC = 2e-2
RMS_FRAC = 1e-2
LSE_ABS = 2e-2
LSE_REL = 4e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _d():
    return torch.device("cuda", 0)


def _log(msg):
    print(msg, flush=True)


def run_train(wl, layer, dout, sinks=None):
    """Forward with lse, then backward, through the C ABI (THD form)."""
    d = _d()
    q, k, v = wl.q.to(d), wl.k.to(d), wl.v.to(d)
    qw, kw = wl.q_norm_w.to(d), wl.k_norm_w.to(d)
    sk = (wl.sinks if sinks is None else torch.as_tensor(sinks, dtype=torch.float32)).to(d)
    pos = None if wl.positions is None else wl.positions.to(torch.int32).to(d)
    cu = wl.cu_seqlens.to(d)
    su = None if wl.seqused is None else wl.seqused.to(d)
    kw_args = dict(positions=pos, cu_seqlens=cu, seqused=su, max_seqlen=wl.max_seqlen,
                   window=layer.window, use_rope=layer.use_rope, rope_theta=layer.theta,
                   eps=layer.eps)
    out, lse = fa.flint_attn(q, k, v, qw, kw, sk, return_lse=True, **kw_args)
    do = dout.to(d)
    grads = fa.flint_attn_backward(do, q, k, v, qw, kw, sk, out, lse, **kw_args)
    torch.cuda.synchronize()
    return out, lse, grads


def oracle_bwd(wl, layer, dout, sinks=None, rows=None, keys=None):
    return flint_attention_backward(
        f64(wl.q), f64(wl.k), f64(wl.v), f64(wl.q_norm_w), f64(wl.k_norm_w),
        f64(wl.sinks if sinks is None else torch.as_tensor(sinks)), i64(wl.cu_seqlens),
        f64(dout), seqused=i64(wl.seqused), positions=i64(wl.positions), window=layer.window,
        use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps, rows=rows, keys=keys)


def _grade_tensor(got, ref, ok, what):
    g = np.asarray(got, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    if (~ok).any():
        assert np.all(g[~ok] == 0.0), f"{what}: padded tokens are not exact zeros"
    gv, rv = g[ok], np.asarray(ref, np.float64)[ok]
    if rv.size == 0:
        return 0.0, 0.0
    scale = float(np.max(np.abs(rv)))
    err = np.abs(gv - rv)
    max_frac = float(err.max()) / max(scale, 1e-30)
    rms_frac = float(np.linalg.norm(gv - rv)) / max(float(np.linalg.norm(rv)), 1e-30)
    assert max_frac <= MAX_FRAC, f"{what}: max err {max_frac:.3e} x max|ref| > {MAX_FRAC}"
    assert rms_frac <= RMS_FRAC, f"{what}: rms err {rms_frac:.3e} x |ref| > {RMS_FRAC}"
    return max_frac, rms_frac


def _grade_param(got, ref, what):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    tol = 1e-2 * 4.0 * float(np.sum(np.abs(r))) / max(r.size, 1) + 1e-6
    err = float(np.max(np.abs(g - r)))
    assert err <= max(tol, 1e-2 * float(np.max(np.abs(r)))), f"{what}: max err {err:.3e} > {tol:.3e}"
    return err / max(float(np.max(np.abs(r))), 1e-30)


def check_backward(wl, layer, what, sinks=None, dout_std=1.0):
    dout = draw_dout(wl.seed, wl.total_tokens, dout_std)
    _log(f"[bwd] {what}: T={wl.total_tokens} window={layer.window} rope={layer.use_rope}")
    out, lse, (dq, dk, dv, dqw, dkw, dsk) = run_train(wl, layer, dout, sinks)
    ref = oracle_bwd(wl, layer, dout, sinks)
    ok = valid_rows(wl)
    # the normalizer
    lg = lse.float().cpu().numpy().astype(np.float64)
    lr = ref["lse"]
    assert np.all(np.isneginf(lg[~ok])), f"{what}: padded lse is not -inf"
    lerr = float(np.max(np.abs(lg[ok] - lr[ok]) / (LSE_ABS + LSE_REL * np.abs(lr[ok])))) \
        if ok.any() else 0.0
    assert lerr <= 1.0, f"{what}: lse error {lerr:.3f} of its bound"
    stats = {"lse": lerr}
    for name, got, key in (("dq", dq, "dq"), ("dk", dk, "dk"), ("dv", dv, "dv")):
        stats[name] = _grade_tensor(to_np(got), ref[key], ok, f"{what} {name}")
    stats["dq_norm_w"] = _grade_param(dqw.cpu().numpy(), ref["dq_norm_w"], f"{what} dq_norm_w")
    stats["dk_norm_w"] = _grade_param(dkw.cpu().numpy(), ref["dk_norm_w"], f"{what} dk_norm_w")
    stats["dsink"] = _grade_param(dsk.cpu().numpy(), ref["dsink"], f"{what} dsink")
    _log(f"[bwd] {what}: " + ", ".join(
        f"{k} {v[0]:.2e}/{v[1]:.2e}" if isinstance(v, tuple) else f"{k} {v:.2e}"
        for k, v in stats.items()))
    return stats


CASES = [
    ("one tile sliding", make_custom(301, [40]), SLIDING),
    ("ragged documents sliding", make_custom(302, [300, 1, 650, 64, 129]), SLIDING),
    ("two key blocks full", make_custom(303, [257]), FULL),
    ("long sliding past the window", make_custom(304, [1200]), SLIDING),
    ("bshd padding full", make_custom(305, [320, 320, 320], layout="bshd", seqused=[320, 77, 0]),
     FULL),
    ("bshd padding sliding", make_custom(306, [200, 200], layout="bshd", seqused=[133, 200]),
     SLIDING),
    ("random positions theta 1e4", make_custom(307, [700, 90], positions="random"),
     Layer(window=513, use_rope=True, theta=1.0e4)),
    ("window 9", make_custom(308, [400]), Layer(window=9, use_rope=True)),
    ("window 1", make_custom(309, [150]), Layer(window=1, use_rope=False)),
    ("full rope", make_custom(310, [600]), Layer(window=0, use_rope=True)),
    ("norm x1.6", make_custom(311, [500], norm_scale=1.6), SLIDING),
    ("positions beyond 2^24", huge_positions(make_custom(312, [260, 90])), SLIDING),
]


@pytest.mark.parametrize("what,wl,layer", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(what, wl, layer):
    check_backward(wl, layer, what)


@pytest.mark.parametrize("kind", ["minus_inf", "plus_80", "strong"])
def test_backward_sinks(kind):
    wl = make_custom(320, [300, 45], sink_std=6.0)
    s = wl.sinks.clone()
    if kind == "minus_inf":
        s[:] = -float("inf")
    elif kind == "plus_80":
        s[::2] = 80.0
    stats = check_backward(wl, SLIDING, f"sinks {kind}", sinks=s)
    if kind == "minus_inf":
        assert stats["dsink"] == 0.0 or np.isfinite(stats["dsink"])


def test_backward_deterministic():
    wl = make_custom(321, [900, 333])
    dout = draw_dout(wl.seed, wl.total_tokens)
    a = run_train(wl, FULL, dout)[2]
    b = run_train(wl, FULL, dout)[2]
    for x, y in zip(a, b):
        assert torch.equal(x, y), "two identical calls differ"


def test_backward_deterministic_across_waves():
    """Repeated calls give the same bits when the schedule's list of
    equal-cost query blocks (376 here) spans several waves of the schedule
    block, whose order in the list varies from call to call."""
    wl = make_custom(322, [1500] * 8)
    dout = draw_dout(wl.seed, wl.total_tokens)
    runs = [run_train(wl, SLIDING, dout)[2] for _ in range(5)]
    names = ("dq", "dk", "dv", "dq_norm_w", "dk_norm_w", "dsink")
    for other in runs[1:]:
        for name, x, y in zip(names, runs[0], other):
            assert torch.equal(x, y), f"{name} differs between two identical calls"


def test_backward_empty():
    d = _d()
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device=d)  # noqa: E731
    q, k, v = z(0, 32, 128), z(0, 4, 128), z(0, 4, 128)
    w = torch.ones(128, dtype=torch.float32, device=d)
    sk = torch.zeros(32, dtype=torch.float32, device=d)
    cu = torch.zeros(1, dtype=torch.int32, device=d)
    lse = torch.zeros(0, 32, dtype=torch.float32, device=d)
    dq, dk, dv, dqw, dkw, dsk = fa.flint_attn_backward(z(0, 32, 128), q, k, v, w, w, sk, z(0, 32, 128),
                                                       lse, cu_seqlens=cu, max_seqlen=0)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.count_nonzero(dqw).item() == 0
    assert torch.count_nonzero(dkw).item() == 0 and torch.count_nonzero(dsk).item() == 0


def _sample(T, n, seed, edges):
    rng = np.random.default_rng(seed)
    pick = set(range(min(T, 8))) | set(range(max(0, T - 8), T)) | {e for e in edges if e < T}
    pick |= set(rng.integers(0, T, size=n).tolist())
    return np.array(sorted(pick), np.int64)


def test_backward_full_size_sampled():
    """The full-attention layer at 8192 tokens: sampled dq rows and dk/dv keys, dsink exact."""
    wl = make_workload("tstar")
    layer = wl.layers[0]
    dout = draw_dout(wl.seed, wl.total_tokens)
    _log(f"[bwd] full size {wl.name}: T={wl.total_tokens}")
    out, lse, (dq, dk, dv, dqw, dkw, dsk) = run_train(wl, layer, dout)
    rows = _sample(wl.total_tokens, 48, 11, (63, 64, 127, 128, 4095, 4096))
    keys = _sample(wl.total_tokens, 48, 12, (63, 64, 127, 128, 4095, 4096))
    ref = oracle_bwd(wl, layer, dout, rows=rows, keys=keys)
    ok = np.ones(len(rows), bool)
    st = {"dq": _grade_tensor(to_np(dq[torch.as_tensor(rows, device=dq.device)]), ref["dq"], ok, "dq"),
          "dk": _grade_tensor(to_np(dk[torch.as_tensor(keys, device=dk.device)]), ref["dk"],
                              np.ones(len(keys), bool), "dk"),
          "dv": _grade_tensor(to_np(dv[torch.as_tensor(keys, device=dv.device)]), ref["dv"],
                              np.ones(len(keys), bool), "dv"),
          "dsink": _grade_param(dsk.cpu().numpy(), ref["dsink"], "dsink")}
    # the logit-scale identity <w_q, dw_q> = <w_k, dw_k> holds for the gradients at any size
    a = float(torch.dot(wl.q_norm_w, dqw.cpu()))
    b = float(torch.dot(wl.k_norm_w, dkw.cpu()))
    assert abs(a - b) <= 2e-2 * max(abs(a), abs(b)), f"<w_q,dw_q> {a} vs <w_k,dw_k> {b}"
    _log(f"[bwd] full size: {st}, <w,dw> {a:.4g} / {b:.4g}")


def _sub_oracle(wl, layer, dout, s, a, b, rows, keys):
    """The oracle on tokens [a, b) of sequence s, taken as a sequence of its
    own with their positions in s. Returns the oracle's dict for the local
    row and key indices (rows / keys minus a).

    In a sliding layer a row t depends only on keys t - W + 1 .. t and key j
    only on the queries j .. j + W - 1 and their key sets, so a row with
    t - W + 1 >= a (or a = 0) and a key with j - W + 1 >= a (or a = 0) whose
    later valid queries all lie below b get exactly their values in the whole
    sequence; a whole document (a = 0, b = its length) does so in any layer.
    """
    cu = i64(wl.cu_seqlens)
    g0 = int(cu[s])
    L = int(cu[s + 1]) - g0
    u = L if wl.seqused is None else int(i64(wl.seqused)[s])
    pos = (np.arange(L, dtype=np.int64) if wl.positions is None
           else i64(wl.positions)[g0:g0 + L])
    sl = slice(g0 + a, g0 + b)
    return flint_attention_backward(
        f64(wl.q[sl]), f64(wl.k[sl]), f64(wl.v[sl]), f64(wl.q_norm_w), f64(wl.k_norm_w),
        f64(wl.sinks), np.array([0, b - a], np.int64), f64(dout[sl]),
        seqused=np.array([max(0, min(u, b) - a)], np.int64), positions=pos[a:b],
        window=layer.window, use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps,
        rows=np.asarray(rows, np.int64) - a, keys=np.asarray(keys, np.int64) - a)


def _check_pieces(wl, layer, name, pieces):
    """Runs the layer's forward and backward on the whole workload (the
    benchmark's launch configuration) and grades dq rows, dk / dv keys and
    the row normalizer of each piece (s, a, b, rows, keys) against the
    oracle on that piece alone. Padded tokens must get exact zeros."""
    dout = draw_dout(wl.seed, wl.total_tokens)
    _log(f"[bwd] {name} {layer.name}: T={wl.total_tokens}, {len(pieces)} pieces")
    out, lse, (dq, dk, dv, dqw, dkw, dsk) = run_train(wl, layer, dout)
    cu = i64(wl.cu_seqlens)
    for s, a, b, rows, keys in pieces:
        L = int(cu[s + 1] - cu[s])
        u = L if wl.seqused is None else int(i64(wl.seqused)[s])
        rows = np.asarray(sorted(set(rows)), np.int64)
        keys = np.asarray(sorted(set(keys)), np.int64)
        assert rows.min() >= a and rows.max() < b and keys.min() >= a and keys.max() < b
        what = f"{name} {layer.name} seq {s} [{a}, {b})"
        _log(f"[bwd] {what}: {len(rows)} rows, {len(keys)} keys")
        ref = _sub_oracle(wl, layer, dout, s, a, b, rows[rows < u], keys[keys < u])
        gr = torch.as_tensor(int(cu[s]) + rows, device=dq.device)
        gk = torch.as_tensor(int(cu[s]) + keys, device=dq.device)
        vr, vk = rows < u, keys < u
        got_dq, got_dk, got_dv = to_np(dq[gr]), to_np(dk[gk]), to_np(dv[gk])
        assert np.all(got_dq[~vr] == 0.0), f"{what}: padded dq rows are not zeros"
        assert np.all(got_dk[~vk] == 0.0) and np.all(got_dv[~vk] == 0.0), \
            f"{what}: padded dk / dv keys are not zeros"
        st = {"dq": _grade_tensor(got_dq[vr], ref["dq"], np.ones(vr.sum(), bool), f"{what} dq"),
              "dk": _grade_tensor(got_dk[vk], ref["dk"], np.ones(vk.sum(), bool), f"{what} dk"),
              "dv": _grade_tensor(got_dv[vk], ref["dv"], np.ones(vk.sum(), bool), f"{what} dv")}
        lg = lse[gr].float().cpu().numpy().astype(np.float64)
        lr = ref["lse"][rows[vr] - a]
        assert np.all(np.isneginf(lg[~vr])), f"{what}: padded lse is not -inf"
        lerr = float(np.max(np.abs(lg[vr] - lr) / (LSE_ABS + LSE_REL * np.abs(lr))))
        assert lerr <= 1.0, f"{what}: lse error {lerr:.3f} of its bound"
        _log(f"[bwd] {what}: " + ", ".join(f"{k} {v[0]:.2e}/{v[1]:.2e}" for k, v in st.items())
             + f", lse {lerr:.2f} of bound")
    a = float(torch.dot(wl.q_norm_w, dqw.cpu()))
    b = float(torch.dot(wl.k_norm_w, dkw.cpu()))
    assert abs(a - b) <= 2e-2 * max(abs(a), abs(b)), f"<w_q,dw_q> {a} vs <w_k,dw_k> {b}"


def _pick(lo, hi, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    pick = set(range(lo, min(hi, lo + 6))) | set(range(max(lo, hi - 6), hi))
    pick |= {e for e in extra if lo <= e < hi}
    pick |= set(rng.integers(lo, hi, size=n).tolist())
    return sorted(pick)


def test_backward_sliding_full_size_pieces():
    """8 x 8192 tokens with trailing padding, sliding window 513 with RoPE (the
    backward benchmark's sliding workload), graded on three pieces: a
    sequence's first 1,600 tokens, an interior stretch, and the end of the
    most padded sequence with its padding."""
    wl = make_workload("c3")
    layer = wl.layers[0]
    W = layer.window
    u6 = int(i64(wl.seqused)[6])
    a6 = u6 - 1600
    pieces = [
        (0, 0, 1600, _pick(0, 1600, 40, 21, (63, 64, 511, 512, 513)),
         _pick(0, 1600 - W, 40, 22, (63, 64, 511, 512))),
        (3, 2900, 4700, _pick(2900 + W - 1, 4700, 40, 23, (4095, 4096)),
         _pick(2900 + W - 1, 4700 - W, 40, 24, (4095, 4096))),
        (6, a6, 8192, _pick(a6 + W - 1, 8192, 40, 25, (u6 - 1, u6, 8191)),
         _pick(a6 + W - 1, 8192, 40, 26, (u6 - 1, u6, 8191))),
    ]
    _check_pieces(wl, layer, "c3", pieces)


@functools.lru_cache(maxsize=1)
def _c4():
    return make_workload("c4")


@pytest.mark.parametrize("li", [0, 1], ids=["sliding", "full"])
def test_backward_thd_documents_full_size(li):
    """16 THD documents of 135 to 7,525 tokens (both layer kinds): three short
    documents graded whole, and for the sliding layer an interior stretch of
    the longest one."""
    wl = _c4()
    layer = wl.layers[li]
    lens = np.diff(i64(wl.cu_seqlens))
    pieces = []
    for s in (1, 2, 13):
        L = int(lens[s])
        pieces.append((s, 0, L, _pick(0, L, 24, 30 + s), _pick(0, L, 24, 50 + s)))
    if layer.window:
        W = layer.window
        pieces.append((10, 3000, 4800, _pick(3000 + W - 1, 4800, 32, 71),
                       _pick(3000 + W - 1, 4800 - W, 32, 72)))
    _check_pieces(wl, layer, "c4", pieces)
