"""GPU: seeded randomized layouts against the oracles.

Each case draws its own sequence packing, padding, window, RoPE flag,
positions, sink spread and norm scale from a seeded generator, so the grid of
hand-picked cases elsewhere is complemented by combinations nobody chose.
The bars are the same as for the hand-picked cases of each path.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import flint_attention_bshd
from workload import Layer, make_custom

from .common import f64
from .gpu_common import check_against_oracle

pytestmark = pytest.mark.gpu

WINDOWS = [0, 1, 2, 63, 64, 65, 100, 513]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _random_thd(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    lengths = [int(x) for x in rng.integers(1, 701, n)]
    seqused = [int(rng.integers(0, L + 1)) if rng.random() < 0.3 else L for L in lengths]
    positions = ["local", "random", "none"][int(rng.integers(0, 3))]
    wl = make_custom(seed, lengths, layout="thd", seqused=seqused, positions=positions,
                     sink_std=float(rng.uniform(0.5, 4.0)), norm_scale=float(rng.uniform(0.5, 1.8)))
    layer = Layer(window=int(rng.choice(WINDOWS)), use_rope=bool(rng.random() < 0.6))
    return wl, layer, f"n={n} T={sum(lengths)} window={layer.window} rope={layer.use_rope} pos={positions}"


@pytest.mark.parametrize("seed", list(range(7000, 7010)))
def test_random_thd_forward(seed):
    wl, layer, what = _random_thd(seed)
    _log(f"[gpu] random THD {seed}: {what}")
    stats, _ = check_against_oracle(wl, layer)
    _log(f"      {stats}")


@pytest.mark.parametrize("seed", list(range(7100, 7108)))
def test_random_bshd_documents(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    S = int(rng.integers(1, 501))
    ids = np.zeros((B, S), np.int32)
    mask = np.ones((B, S), np.uint8)
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, S), size=min(S - 1, int(rng.integers(0, 6))), replace=False)) \
            if S > 1 else np.array([], int)
        ids[b] = np.searchsorted(cuts, np.arange(S), side="right") + 10 * b
        kind = int(rng.integers(0, 4))
        if kind == 1:
            mask[b, :int(rng.integers(0, S + 1))] = 0  # leading padding
        elif kind == 2:
            mask[b, S - int(rng.integers(0, S + 1)):] = 0  # trailing padding
        elif kind == 3:
            mask[b, rng.random(S) < float(rng.uniform(0.02, 0.4))] = 0  # holes
    wl = make_custom(seed, [S] * B, layout="bshd", norm_scale=float(rng.uniform(0.6, 1.5)))
    layer = Layer(window=int(rng.choice(WINDOWS)), use_rope=bool(rng.random() < 0.6))
    d = torch.device("cuda", 0)
    _log(f"[gpu] random BSHD {seed}: B={B} S={S} window={layer.window} rope={layer.use_rope} "
         f"valid={int(mask.sum())}")
    out = fa.flint_attn(wl.q.to(d).view(B, S, 32, 128), wl.k.to(d).view(B, S, 4, 128),
                        wl.v.to(d).view(B, S, 4, 128), wl.q_norm_w.to(d), wl.k_norm_w.to(d),
                        wl.sinks.to(d), attention_mask=torch.from_numpy(mask).to(d),
                        document_ids=torch.from_numpy(ids).to(d), window=layer.window,
                        use_rope=layer.use_rope)
    torch.cuda.synchronize()
    ref = flint_attention_bshd(f64(wl.q).reshape(B, S, 32, 128), f64(wl.k).reshape(B, S, 4, 128),
                               f64(wl.v).reshape(B, S, 4, 128), f64(wl.q_norm_w),
                               f64(wl.k_norm_w), f64(wl.sinks), attention_mask=mask,
                               document_ids=ids, window=layer.window, use_rope=layer.use_rope)
    got = out.float().cpu().numpy().astype(np.float64)
    ok = mask != 0
    vmax = float(np.abs(f64(wl.v)).max())
    assert np.all(got[~ok] == 0.0), "padded rows are not zeros"
    if ok.any():
        err = np.abs(got[ok] - ref[ok])
        _log(f"      max_frac {err.max() / vmax:.3g} mean_frac {err.mean() / vmax:.3g}")
        assert err.max() <= 2e-2 * vmax and err.mean() <= 1e-3 * vmax


@pytest.mark.parametrize("seed", list(range(7200, 7205)))
def test_random_backward(seed):
    from .test_gpu_backward import check_backward

    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(1, 400, n)]
    seqused = [int(rng.integers(0, L + 1)) if rng.random() < 0.3 else L for L in lengths]
    wl = make_custom(seed, lengths, layout="thd", seqused=seqused,
                     positions=["local", "random"][int(rng.integers(0, 2))],
                     sink_std=float(rng.uniform(0.5, 3.0)))
    layer = Layer(window=int(rng.choice(WINDOWS)), use_rope=bool(rng.random() < 0.6))
    check_backward(wl, layer, f"random {seed} n={n} T={sum(lengths)} window={layer.window}")


@pytest.mark.parametrize("seed", list(range(7300, 7304)))
def test_random_decode(seed):
    from .test_gpu_decode import _decode_and_check

    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    window = int(rng.choice([0, 64, 513]))
    layer = Layer(window=window, use_rope=window > 0 or bool(rng.random() < 0.5))
    prefix = [int(x) for x in rng.integers(0, 1500, B)]
    steps = 2
    wl = make_custom(seed, [p + steps for p in prefix], layers=(layer,),
                     positions=["local", "random"][int(rng.integers(0, 2))],
                     sink_std=float(rng.uniform(0.5, 3.0)))
    cap = 0 if window > 0 else max(prefix) + steps + 32
    _decode_and_check(wl, layer, prefix, steps, cap, f"random {seed} B={B} window={window}")


@pytest.mark.parametrize("seed", list(range(7400, 7404)))
def test_random_fp16_forward(seed):
    from .test_gpu_fp16 import check

    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    lengths = [int(x) for x in rng.integers(1, 600, n)]
    wl = make_custom(seed, lengths, layout="thd", dtype="float32",
                     positions=["local", "random", "none"][int(rng.integers(0, 3))],
                     norm_scale=float(rng.uniform(0.3, 2.0)))
    layer = Layer(window=int(rng.choice(WINDOWS)), use_rope=bool(rng.random() < 0.6))
    _log(f"[gpu] random FP16 {seed}: n={n} T={sum(lengths)} window={layer.window} rope={layer.use_rope}")
    check(wl, layer, what=f"random fp16 {seed}")
