"""GPU: one sequence of FLINT_MAX_SEQLEN tokens (2^21), the longest the prefill takes.

At this size the host cannot hold FP64 copies of the inputs, so the checks are
built to need none:
- the sliding RoPE layer is checked row by row against the oracle on each
  sampled row's own window (its 513 keys with their true positions), which is
  the whole of what that row depends on;
- the full NoPE layer uses inputs whose answer has a closed form at any size:
  zero queries make every logit 0, so with a sink of -inf every row averages
  the values of its keys 0..t uniformly. Value channels set to a ramp, ones and
  an alternating sign then give prefix means, ones and (0 or 1/(t+1)). Wrong
  tile data or offsets along the 32,768 key tiles of the last rows show in
  them; per-row parity at long lengths is the 131,072-token sampled test.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import flint_attention
from workload import draw_large, draw_large_params

from .common import f64

pytestmark = pytest.mark.gpu

T = 1 << 21  # FLINT_MAX_SEQLEN of include/flint_attn.h


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()
    yield
    torch.cuda.empty_cache()


def _log(msg):
    print(msg, flush=True)


def test_max_seqlen_sliding_rope_rows():
    d = torch.device("cuda", 0)
    _log(f"[gpu] max seqlen sliding RoPE: one sequence of {T} tokens")
    q, k, v = draw_large(2021, T, d)
    qw, kw, sk = draw_large_params(2021)
    cu = torch.tensor([0, T], dtype=torch.int32, device=d)
    out = fa.flint_attn(q, k, v, qw.to(d), kw.to(d), sk.to(d), cu_seqlens=cu, max_seqlen=T,
                        window=513, use_rope=True)
    torch.cuda.synchronize()
    vmax = float(v.abs().max())
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 63, 64, 511, 512, 513, 4095, 1 << 20, (1 << 20) + 31, T - 64, T - 33,
                   T - 32, T - 1} | {int(x) for x in rng.integers(0, T, 26)})
    errs = []
    for t in rows:
        lo = max(0, t - 512)
        ref = flint_attention(f64(q[lo:t + 1].cpu()), f64(k[lo:t + 1].cpu()), f64(v[lo:t + 1].cpu()),
                              f64(qw), f64(kw), f64(sk), np.array([0, t + 1 - lo]),
                              positions=np.arange(lo, t + 1), window=513, use_rope=True,
                              rows=[t - lo])[0]
        errs.append(np.abs(out[t].float().cpu().numpy().astype(np.float64) - ref))
    e = np.stack(errs)
    _log(f"      rows {len(rows)} max_frac {e.max() / vmax:.3g} mean_frac {e.mean() / vmax:.3g}")
    assert e.max() <= 2e-2 * vmax and e.mean() <= 1e-3 * vmax
    del q, k, v, out


def test_max_seqlen_full_uniform_weights():
    d = torch.device("cuda", 0)
    _log(f"[gpu] max seqlen full NoPE, closed form: one sequence of {T} tokens")
    q = torch.zeros(T, 32, 128, dtype=torch.bfloat16, device=d)
    k = draw_large(2022, T, d)[1]
    j = torch.arange(T, device=d)
    ramp = (j.double() / T).to(torch.bfloat16)
    alt = (1 - 2 * (j % 2)).to(torch.bfloat16)
    v = torch.zeros(T, 4, 128, dtype=torch.bfloat16, device=d)
    v[:, :, 0] = ramp[:, None]
    v[:, :, 1] = 1.0
    v[:, :, 2] = alt[:, None]
    qw, kw, _ = draw_large_params(2022)
    sk = torch.full((32,), float("-inf"), dtype=torch.float32, device=d)
    cu = torch.tensor([0, T], dtype=torch.int32, device=d)
    out = fa.flint_attn(q, k, v, qw.to(d), kw.to(d), sk, cu_seqlens=cu, max_seqlen=T, window=0,
                        use_rope=False)
    torch.cuda.synchronize()
    del q, k
    cnt = (j + 1).double()
    exp_ramp = torch.cumsum(ramp.double(), 0) / cnt
    exp_alt = torch.cumsum(alt.double(), 0) / cnt
    assert bool((out[:, :, 1] == 1).all()), "the weights of a row do not sum to 1"
    assert bool((out[:, :, 3:] == 0).all())
    # Relative bound: the bf16 output rounding (2^-9) plus FP32 accumulation of
    # up to 2^17 tile-step partial sums (4 per 64-key tile) into the running
    # output, each add off by at most one unit in the last place (2^-23) when
    # the matrix cores do not round to nearest: 2^17 * 2^-23 = 2^-6. Measured:
    # 3.9e-3 on the ramp at 2^21 keys, output rounding included.
    rel = 2.0 ** -9 + 2.0 ** -6
    e0 = (out[:, :, 0].double() - exp_ramp[:, None]).abs()
    e2 = (out[:, :, 2].double() - exp_alt[:, None]).abs()
    tol0 = rel * exp_ramp[:, None] + 1e-9
    tol2 = rel * exp_alt[:, None].abs() + 1e-9
    _log(f"      ramp max rel {float((e0 / (exp_ramp[:, None] + 1e-30)).max()):.3g}, "
         f"alternating max abs {float(e2.max()):.3g}")
    assert bool((e0 <= tol0).all()) and bool((e2 <= tol2).all())
    del v, out


def test_max_seqlen_sliding_rope_backward_pieces():
    """The backward of the sliding RoPE layer at 2^21 tokens, graded on three
    stretches the oracle takes alone (with their true positions): a sliding
    row depends only on its 513 keys and a key only on the 513 queries after
    it, so rows and keys at least 512 tokens inside a stretch get their
    whole-sequence gradients. The logit-scale identity <w_q, dw_q> =
    <w_k, dw_k> holds for the weight gradients at any size."""
    from oracle import flint_attention_backward

    d = torch.device("cuda", 0)
    W = 513
    _log(f"[gpu] max seqlen sliding RoPE backward: one sequence of {T} tokens")
    q, k, v = draw_large(2023, T, d)
    dout = draw_large(2024, T, d)[0]
    qw, kw, sk = draw_large_params(2023)
    cu = torch.tensor([0, T], dtype=torch.int32, device=d)
    kwargs = dict(cu_seqlens=cu, max_seqlen=T, window=W, use_rope=True)
    out, lse = fa.flint_attn(q, k, v, qw.to(d), kw.to(d), sk.to(d), return_lse=True, **kwargs)
    dq, dk, dv, dqw, dkw, dsk = fa.flint_attn_backward(dout, q, k, v, qw.to(d), kw.to(d), sk.to(d), out, lse,
                                                       **kwargs)
    torch.cuda.synchronize()
    del out, lse
    rng = np.random.default_rng(8)
    worst = {}
    for a, b in ((0, 1600), ((1 << 20) - 800, (1 << 20) + 1000), (T - 1800, T)):
        r0 = a + W - 1 if a > 0 else 0
        k1 = b - W + 1 if b < T else T
        rows = sorted({r0, r0 + 1, b - 1} | {int(x) for x in rng.integers(r0, b, 20)})
        keys = sorted({r0, k1 - 1} | {int(x) for x in rng.integers(r0, k1, 20)})
        _log(f"      stretch [{a}, {b}): {len(rows)} rows, {len(keys)} keys")
        ref = flint_attention_backward(
            f64(q[a:b].cpu()), f64(k[a:b].cpu()), f64(v[a:b].cpu()), f64(qw), f64(kw), f64(sk),
            np.array([0, b - a]), f64(dout[a:b].cpu()), positions=np.arange(a, b), window=W, use_rope=True,
            rows=np.array(rows) - a, keys=np.array(keys) - a)
        for name, got, want in (("dq", dq[torch.as_tensor(rows, device=d)], ref["dq"]),
                                ("dk", dk[torch.as_tensor(keys, device=d)], ref["dk"]),
                                ("dv", dv[torch.as_tensor(keys, device=d)], ref["dv"])):
            g = got.float().cpu().numpy().astype(np.float64)
            scale = float(np.max(np.abs(want)))
            mx = float(np.max(np.abs(g - want))) / scale
            rms = float(np.linalg.norm(g - want) / np.linalg.norm(want))
            worst[name] = max(worst.get(name, 0.0), mx)
            assert mx <= 2e-2 and rms <= 1e-2, f"[{a}, {b}) {name}: max {mx:.3g}, rms {rms:.3g}"
    wa = float(torch.dot(qw, dqw.cpu()))
    wb = float(torch.dot(kw, dkw.cpu()))
    _log(f"      worst max errors {worst}; <w_q,dw_q> {wa:.5g}, <w_k,dw_k> {wb:.5g}")
    assert abs(wa - wb) <= 2e-2 * max(abs(wa), abs(wb))
    assert torch.isfinite(dsk).all()
    del q, k, v, dout, dq, dk, dv
