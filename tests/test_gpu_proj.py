"""GPU: the q/k/v and output projections, and the attention block end to end.

Projections against FP64 products of the same bf16 inputs. The kernel
accumulates in FP32 and rounds once to bf16, so an element may differ from the
exact product by half a bf16 ulp (2^-9 relative) plus the FP32 accumulation
error, bounded by K 2^-24 sum_k |x_k w_k| (written here as 2^-12 sum|x w|,
K <= 4096): |err| <= 2^-8 |ref| + 2^-12 sum_k |x_k w_k|.

The block (projections, layer, output projection) against the block oracle:
the bf16 roundings of q, k, v, of the layer's output and of y, and the layer's
own error, each a few 2^-9 relative, compound to about 1% of |y|; the bars are
mean |err| <= 2e-2 mean |y| and max |err| <= 2e-2 max |y|.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import flint_attention_block, linear
from workload import draw_block, make_custom
from workload.gen import FULL, SLIDING

from .common import f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _check_linear(got, x, w, rows, what):
    """got [len(rows), N] against rows `rows` of x [T, K] times w^T."""
    xr = f64(x[torch.from_numpy(np.asarray(rows))])
    wf = f64(w)
    ref = xr @ wf.T
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * (np.abs(xr) @ np.abs(wf).T)
    g = got.float().cpu().numpy().astype(np.float64).reshape(len(rows), -1)
    err = np.abs(g - ref)
    worst = float((err / np.maximum(bound, 1e-30)).max())
    _log(f"      {what}: max err {err.max():.3g}, worst err / bound {worst:.3f}")
    assert np.all(err <= bound), f"{what}: err above bound (worst ratio {worst:.3f})"


@pytest.mark.parametrize("T", [1, 7, 255, 256, 257, 1000, 3000])
def test_qkv_projection(T):
    x, w_q, w_k, w_v, _ = draw_block(500 + T, T)
    d = torch.device("cuda", 0)
    q, k, v = fa.qkv_projection(x.to(d), w_q.to(d), w_k.to(d), w_v.to(d))
    torch.cuda.synchronize()
    rows = np.arange(T)
    _log(f"[gpu] qkv projection T={T}")
    _check_linear(q.view(T, -1), x, w_q, rows, "q")
    _check_linear(k.view(T, -1), x, w_k, rows, "k")
    _check_linear(v.view(T, -1), x, w_v, rows, "v")


@pytest.mark.parametrize("T", [1, 255, 257, 1000])
def test_output_projection(T):
    _, _, _, _, w_o = draw_block(600 + T, 1)
    o = torch.from_numpy(np.random.default_rng(T).normal(0, 1, (T, 32, 128)).astype(np.float32))
    o = o.bfloat16()
    d = torch.device("cuda", 0)
    y = fa.output_projection(o.to(d), w_o.to(d))
    torch.cuda.synchronize()
    _log(f"[gpu] output projection T={T}")
    _check_linear(y, o.view(T, -1), w_o, np.arange(T), "y")


def test_full_size_sampled():
    """8,192 tokens (the benchmark's size) and 8 x 8,192: sampled rows."""
    d = torch.device("cuda", 0)
    for T in (8192, 65536):
        x, w_q, w_k, w_v, w_o = draw_block(700, T)
        q, k, v = fa.qkv_projection(x.to(d), w_q.to(d), w_k.to(d), w_v.to(d))
        y = fa.output_projection(q, w_o.to(d))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(0, T, 257), [T - 1],
                                         np.random.default_rng(T).integers(0, T, 200)]))
        ri = torch.from_numpy(rows).to(d)
        _log(f"[gpu] projections T={T}, {len(rows)} rows")
        _check_linear(q[ri].view(len(rows), -1), x, w_q, rows, "q")
        _check_linear(v[ri].view(len(rows), -1), x, w_v, rows, "v")
        _check_linear(y[ri], q[ri].view(len(rows), -1).cpu(), w_o, np.arange(len(rows)), "y")


def test_matches_torch_linear():
    """Same inputs through torch's linear (hipBLASLt): agreement to the bf16 output rounding."""
    T = 2000
    x, w_q, w_k, w_v, w_o = draw_block(800, T)
    d = torch.device("cuda", 0)
    q, k, v = fa.qkv_projection(x.to(d), w_q.to(d), w_k.to(d), w_v.to(d))
    ref = torch.nn.functional.linear(x.to(d).float(), w_q.to(d).float())
    torch.cuda.synchronize()
    err = (q.view(T, -1).float() - ref).abs()
    assert float(err.max()) <= 2.0 ** -7 * float(ref.abs().max())


@pytest.mark.parametrize("layer,lengths", [(SLIDING, [300, 700, 1]), (FULL, [513, 257])],
                         ids=["sliding", "full"])
def test_block_against_oracle(layer, lengths):
    wl = make_custom(900 + len(lengths), lengths)
    T = wl.total_tokens
    x, w_q, w_k, w_v, w_o = draw_block(900, T)
    d = torch.device("cuda", 0)
    y = fa.flint_attention_block(x.to(d), w_q.to(d), w_k.to(d), w_v.to(d), w_o.to(d),
                                 wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d),
                                 cu_seqlens=wl.cu_seqlens.to(d), max_seqlen=wl.max_seqlen,
                                 window=layer.window, use_rope=layer.use_rope)
    torch.cuda.synchronize()
    ref, _, _ = flint_attention_block(f64(x), f64(w_q), f64(w_k), f64(w_v), f64(w_o),
                                      f64(wl.q_norm_w), f64(wl.k_norm_w), f64(wl.sinks),
                                      wl.cu_seqlens.numpy().astype(np.int64), window=layer.window,
                                      use_rope=layer.use_rope)
    g = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    _log(f"[gpu] block {layer.name}: mean err / mean|y| {err.mean() / np.abs(ref).mean():.3g}, "
         f"max err / max|y| {err.max() / np.abs(ref).max():.3g}")
    assert err.mean() <= 2e-2 * np.abs(ref).mean()
    assert err.max() <= 2e-2 * np.abs(ref).max()
