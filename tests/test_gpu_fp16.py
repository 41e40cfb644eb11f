"""GPU parity of the FP16 attention-compute variant against the FP64 oracle.

The variant (flint page, Numerical comparison: attention_compute_dtype fp16)
takes FP32 projections, runs RMSNorm and RoPE in FP32, rounds q', k' and v to
fp16 once, multiplies on fp16 MFMA with FP32 accumulation and returns FP32
holding the fp16-rounded output. The oracle sees the same FP32 inputs in FP64.

Tolerance, from the arithmetic: fp16 keeps 11 significant bits (unit roundoff
u = 2^-11 ~ 4.9e-4). The output rounding alone moves an element by up to
u |O| <= u max|V|; the rounding of q' and k' moves a logit by about
sqrt(D) |q'_i||k'_i| u / sqrt(D), a relative weight error of order 1e-3 on
the largest logits of these workloads; the fp16 rounding of the softmax
weights and of v adds u each, averaged over the keys. The bars are
max |err| <= 4e-3 max|V| (eight times the output rounding) and
mean |err| <= 2.5e-4 max|V|, ten times tighter than the bfloat16 path's
2e-2 / 1e-3, so a kernel that rounded anything to bfloat16 fails them.
Padded rows must be exact zeros.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from workload import Layer, make_custom, make_workload
from workload.gen import FULL, SLIDING

from .common import f64, i64, oracle_for
from .gpu_common import grade

pytestmark = pytest.mark.gpu

MAX_FRAC = 4e-3
MEAN_FRAC = 2.5e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _fp32(wl):
    """The same workload with float32 projections (bf16 values are exact in FP32)."""
    wl.q, wl.k, wl.v = wl.q.float(), wl.k.float(), wl.v.float()
    return wl


def run_f16(wl, layer, *, sinks=None, bshd=None, workspace=None):
    d = torch.device("cuda", 0)
    q, k, v = wl.q.to(d), wl.k.to(d), wl.v.to(d)
    assert q.dtype == torch.float32
    qw, kw = wl.q_norm_w.to(d), wl.k_norm_w.to(d)
    sk = (wl.sinks if sinks is None else torch.as_tensor(sinks, dtype=torch.float32)).to(d)
    pos = None if wl.positions is None else wl.positions.to(torch.int32).to(d)
    kw_args = dict(window=layer.window, use_rope=layer.use_rope, rope_theta=layer.theta,
                   eps=layer.eps, workspace=workspace)
    if (wl.layout == "bshd") if bshd is None else bshd:
        B, S = wl.batch, wl.seqlen
        mask = wl.attention_mask()
        o = fa.flint_attn_f16(q.view(B, S, 32, 128), k.view(B, S, 4, 128), v.view(B, S, 4, 128),
                              qw, kw, sk, positions=None if pos is None else pos.view(B, S),
                              attention_mask=None if mask is None else mask.to(d), **kw_args)
        return o.view(B * S, 32, 128)
    su = None if wl.seqused is None else wl.seqused.to(d)
    return fa.flint_attn_f16(q, k, v, qw, kw, sk, positions=pos, cu_seqlens=wl.cu_seqlens.to(d),
                             seqused=su, max_seqlen=wl.max_seqlen, **kw_args)


def check(wl, layer, rows=None, sinks=None, what=""):
    out = run_f16(wl, layer, sinks=sinks)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    got = got.cpu().numpy().astype(np.float64)
    # Every output element is an fp16 value held in FP32.
    assert np.array_equal(got, got.astype(np.float16).astype(np.float64)), f"{what}: not fp16 values"
    over = {} if sinks is None else {"sinks": np.asarray(sinks, np.float64)}
    ref = oracle_for(wl, layer, rows=rows, **over)
    stats = grade(got, ref, wl, rows=rows, what=what or f"{wl.name}/{layer.name}",
                  max_frac=MAX_FRAC, mean_frac=MEAN_FRAC)
    _log(f"      {stats}")
    return out


SMALL = [
    ("one tile", make_custom(301, [40], dtype="float32"), SLIDING),
    ("several tiles sliding", make_custom(302, [700], dtype="float32"), SLIDING),
    ("several tiles full", make_custom(303, [333], dtype="float32"), FULL),
    ("ragged THD sliding", make_custom(304, [130, 1, 65, 300, 2], dtype="float32"), SLIDING),
    ("ragged THD full", make_custom(305, [130, 1, 65, 300, 2], dtype="float32"), FULL),
    ("BSHD trailing padding",
     make_custom(306, [256, 256, 256], layout="bshd", seqused=[256, 100, 0], dtype="float32"), SLIDING),
    ("window 1", make_custom(308, [150], dtype="float32"), Layer(window=1, use_rope=True)),
    ("window 65 nope", make_custom(311, [300], dtype="float32"), Layer(window=65, use_rope=False)),
    ("random large positions", make_custom(312, [200], positions="random", dtype="float32"), SLIDING),
    ("strong sinks", make_custom(314, [260], sink_std=6.0, dtype="float32"), FULL),
    ("tiny sequences", make_custom(316, [1, 2, 3, 31, 32, 33, 63, 64, 65], dtype="float32"), SLIDING),
]


@pytest.mark.parametrize("name,wl,layer", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(name, wl, layer):
    _log(f"[gpu] fp16 small parity: {name} seed={wl.seed} T={wl.total_tokens}")
    check(wl, layer, what=name)


@pytest.mark.parametrize("scale", [0.3, 1.6, 2.2])
def test_logit_range_paths(scale):
    """Small logits take the unshifted path (bound under 15 log2 units: fp16
    weights cannot overflow), large ones the streaming running-max path."""
    wl = make_custom(340 + int(scale * 10), [700, 130], norm_scale=scale, dtype="float32")
    _log(f"[gpu] fp16 logit range, norm weights x{scale}")
    for layer in (SLIDING, FULL):
        check(wl, layer, what=f"x{scale} {layer.name}")
        check(wl, layer, sinks=np.full(32, -np.inf, np.float32), what=f"x{scale} {layer.name} -inf")


def test_fp32_inputs_are_used_unrounded():
    """Inputs that bfloat16 cannot hold: the result follows the FP32 values."""
    wl = make_custom(350, [400], dtype="float32")
    rng = np.random.default_rng(350)
    for t in (wl.q, wl.k, wl.v):
        t += torch.from_numpy(rng.normal(0, 1e-3, t.shape).astype(np.float32))
    assert not torch.equal(wl.v, wl.v.bfloat16().float())
    check(wl, FULL, what="unrounded fp32")


def test_deterministic_and_padding_zero():
    wl = make_custom(351, [300, 300], layout="bshd", seqused=[300, 77], dtype="float32")
    a = run_f16(wl, SLIDING)
    b = run_f16(wl, SLIDING, bshd=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.all(a[300 + 77:] == 0)


def test_matches_bf16_path_within_bf16_bar():
    """On bf16-representable inputs the two variants agree to the bf16 bar."""
    wl = make_custom(352, [600])
    d = torch.device("cuda", 0)
    args = (wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d))
    kw = dict(positions=wl.positions.to(torch.int32).to(d), cu_seqlens=wl.cu_seqlens.to(d),
              max_seqlen=600, window=513, use_rope=True)
    o16 = fa.flint_attn_f16(wl.q.float().to(d), wl.k.float().to(d), wl.v.float().to(d), *args, **kw)
    obf = fa.flint_attn(wl.q.to(d), wl.k.to(d), wl.v.to(d), *args, **kw)
    torch.cuda.synchronize()
    vmax = float(wl.v.float().abs().max())
    assert float((o16 - obf.float()).abs().max()) <= 2e-2 * vmax


def test_rejects_bf16_inputs():
    wl = make_custom(353, [64])
    d = torch.device("cuda", 0)
    with pytest.raises(TypeError):
        fa.flint_attn_f16(wl.q.to(d), wl.k.to(d), wl.v.to(d), wl.q_norm_w.to(d), wl.k_norm_w.to(d),
                          wl.sinks.to(d), cu_seqlens=wl.cu_seqlens.to(d), max_seqlen=64)


def test_empty_input():
    d = torch.device("cuda")
    q = torch.empty(0, 32, 128, device=d)
    k = torch.empty(0, 4, 128, device=d)
    w = torch.ones(128, device=d)
    out = fa.flint_attn_f16(q, k, k, w, w, torch.zeros(32, device=d),
                            cu_seqlens=torch.zeros(1, dtype=torch.int32, device=d), max_seqlen=0)
    assert out.shape == (0, 32, 128)


def _rows(wl, per_seq, seed):
    rng = np.random.default_rng(seed)
    cu = i64(wl.cu_seqlens)
    rows = set()
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        u = b - a if wl.seqused is None else int(wl.seqused[s])
        rows |= {a + x for x in range(min(16, b - a))}
        rows |= {a + x for x in range(max(0, u - 8), min(b - a, u + 8))}
        rows |= {a + int(x) for x in rng.integers(0, b - a, per_seq)}
    return np.array(sorted(rows), np.int64)


def test_tstar_sampled():
    wl = _fp32(make_workload("tstar"))
    rows = _rows(wl, 96, 1307)
    _log(f"[gpu] fp16 S=8192 full NoPE sampled rows={len(rows)}")
    check(wl, wl.layers[0], rows=rows, what="tstar fp16")


def test_c3_sampled():
    wl = _fp32(make_workload("c3"))
    rows = _rows(wl, 48, 1304)
    _log(f"[gpu] fp16 B=8 S=8192 sliding sampled rows={len(rows)}")
    check(wl, wl.layers[0], rows=rows, what="c3 fp16")
