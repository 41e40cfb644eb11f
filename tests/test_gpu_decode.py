"""GPU parity of the decode path (KV-cache append + one-token attention) against the oracle.

Decoding token t of a sequence computes row t of the layer over the sequence's
tokens 0..t; the hybrid KV cache only changes where the keys are kept (Hugging
Face discussion #26 on RecursiveSI/flint, "Minor": per-layer window sizes are
honoured, a ring of the last 513 tokens for sliding layers and every token for
full layers). So the oracle is the prefill oracle restricted to that row, and
the cached keys are the oracle's RMSNorm + RoPE of each key.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import rms_norm, rope_neox
from workload import Layer, make_custom, make_long_decode
from workload.gen import FULL, SLIDING

from .common import f64, i64, oracle_for
from .gpu_common import grade, to_np

pytestmark = pytest.mark.gpu


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


def _cache_for(wl, layer, prefix, cap_tokens):
    """A batched cache whose sequence b holds its first prefix[b] tokens.

    Each sequence is filled through its own one-sequence cache (appends of at
    most one ring's worth of tokens), then copied into the batched layout.
    """
    d = _d()
    B = len(prefix)
    cache = fa.KVCache(B, layer.window, max_tokens=cap_tokens, use_rope=layer.use_rope,
                       rope_theta=layer.theta, eps=layer.eps, device=d)
    kw = wl.k_norm_w.to(d)
    cu = i64(wl.cu_seqlens)
    for b in range(B):
        n = int(prefix[b])
        if n == 0:
            continue
        one = fa.KVCache(1, layer.window, max_tokens=cap_tokens, use_rope=layer.use_rope,
                         rope_theta=layer.theta, eps=layer.eps, device=d)
        chunk = one.cap if layer.window > 0 else n
        s0 = int(cu[b])
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            k = wl.k[s0 + c0:s0 + c1].unsqueeze(0).contiguous().to(d)
            v = wl.v[s0 + c0:s0 + c1].unsqueeze(0).contiguous().to(d)
            pos = None
            if wl.positions is not None:
                pos = wl.positions[s0 + c0:s0 + c1].view(1, -1).contiguous().to(d)
            one.append(k, v, kw, pos)
        cache.k[b] = one.k[0]
        cache.vt[b] = one.vt[0]
        cache.length[b] = n
    torch.cuda.synchronize()
    return cache


def _decode_and_check(wl, layer, prefix, steps, cap_tokens, what, sinks=None):
    """Runs `steps` decode steps after the prefixes and grades every step against the oracle."""
    d = _d()
    cache = _cache_for(wl, layer, prefix, cap_tokens)
    cu = i64(wl.cu_seqlens)
    qw, kw = wl.q_norm_w.to(d), wl.k_norm_w.to(d)
    sk = (wl.sinks if sinks is None else torch.as_tensor(sinks, dtype=torch.float32)).to(d)
    worst = 0.0
    for j in range(steps):
        rows = np.array([int(cu[b]) + int(prefix[b]) + j for b in range(len(prefix))])
        idx = torch.as_tensor(rows)
        q = wl.q[idx].contiguous().to(d)
        k = wl.k[idx].contiguous().to(d)
        v = wl.v[idx].contiguous().to(d)
        pos = None if wl.positions is None else wl.positions[idx].contiguous().to(d)
        _log(f"[decode] {what}: step {j}, lengths {[int(p) + j for p in prefix]}")
        out = cache.decode(q, k, v, qw, kw, sk, pos)
        st, flags = cache.device_status()
        assert st == fa.FLINT_OK and flags == 0, (st, flags)
        ref = oracle_for(wl, layer, rows=rows, sinks=f64(sk.cpu()))
        stats = grade(to_np(out), ref, wl, rows=rows, what=f"{what} step {j}")
        worst = max(worst, stats["max_frac"])
    _log(f"[decode] {what}: worst max err {worst:.3e} x max|V|")
    return cache


def test_full_layer_mixed_lengths():
    # block edges (31, 32, 33), split edges (255, 256, 257), a long one
    prefix = [0, 1, 31, 32, 33, 255, 256, 257, 1000, 2049]
    steps = 3
    wl = make_custom(4001, [p + steps for p in prefix], layers=(FULL,))
    _decode_and_check(wl, FULL, prefix, steps, 2080, "full mixed")


def test_sliding_layer_ring_wrap():
    # shorter than the window, at the window, past the ring capacity (544)
    prefix = [0, 100, 511, 512, 513, 514, 543, 544, 600, 1100, 1631]
    steps = 3
    wl = make_custom(4002, [p + steps for p in prefix], layers=(SLIDING,))
    _decode_and_check(wl, SLIDING, prefix, steps, 0, "sliding ring")


def test_random_positions_and_theta():
    layer = Layer(window=513, use_rope=True, theta=1.0e4)
    prefix = [3, 700, 1200]
    wl = make_custom(4003, [p + 2 for p in prefix], layers=(layer,), positions="random")
    _decode_and_check(wl, layer, prefix, 2, 0, "random positions theta 1e4")


@pytest.mark.parametrize("kind", ["minus_inf", "plus_80", "strong"])
def test_sinks(kind):
    prefix = [0, 40, 300]
    wl = make_custom(4004, [p + 2 for p in prefix], layers=(FULL,), sink_std=6.0)
    s = wl.sinks.clone()
    if kind == "minus_inf":
        s[:] = -float("inf")
    elif kind == "plus_80":
        s[::2] = 80.0
    _decode_and_check(wl, FULL, prefix, 2, 352, f"sinks {kind}", sinks=s)


def test_large_logits():
    prefix = [64, 500]
    wl = make_custom(4005, [p + 2 for p in prefix], layers=(SLIDING,), norm_scale=1.6)
    _decode_and_check(wl, SLIDING, prefix, 2, 0, "norm x1.6")


def test_cache_contents_match_oracle_keys():
    """K' rows are the oracle's RMSNorm + RoPE of k rounded to bf16; V holds v exactly
    (both read back through the block layout the header documents)."""
    layer = SLIDING
    n = 700  # wraps the 544-slot ring: slots hold tokens 156..699
    wl = make_custom(4006, [n], layers=(layer,), positions="random")
    cache = _cache_for(wl, layer, [n], 0)
    kref = rope_neox(rms_norm(f64(wl.k), f64(wl.k_norm_w), layer.eps), f64(wl.positions),
                     layer.theta)  # [n, 4, 128]
    cap = cache.cap
    tok = np.arange(n - cap, n)
    slots = tok % cap
    got_k = cache.dense_keys()[0].float().cpu().numpy().astype(np.float64)[:, slots, :]  # [4, n, 128]
    ref_k = kref[tok].transpose(1, 0, 2)
    err = np.abs(got_k - ref_k)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref_k) + 1e-6), f"K' max err {err.max():.3g}"
    got_v = cache.dense_values()[0].cpu()[:, torch.as_tensor(slots), :]  # [4, n, 128]
    ref_v = wl.v[torch.as_tensor(tok)].permute(1, 0, 2)
    assert torch.equal(got_v, ref_v)


def test_full_cache_overflow_reported_and_zero_output():
    d = _d()
    wl = make_custom(4007, [40], layers=(FULL,))
    cache = _cache_for(wl, FULL, [32], 32)  # full: the 33rd token does not fit
    q, k, v = wl.q[32:33].to(d), wl.k[32:33].to(d), wl.v[32:33].to(d)
    out = cache.decode(q.contiguous(), k.contiguous(), v.contiguous(), wl.q_norm_w.to(d),
                       wl.k_norm_w.to(d), wl.sinks.to(d))
    st, flags = cache.device_status()
    assert st == fa.FLINT_ERR_DEVICE_DATA and flags & fa.FLINT_DEV_CACHE
    assert torch.count_nonzero(out).item() == 0


def test_decode_argument_errors():
    d = _d()
    cache = fa.KVCache(2, 513)
    q = torch.zeros(2, 32, 128, dtype=torch.bfloat16, device=d)
    k = torch.zeros(2, 4, 128, dtype=torch.bfloat16, device=d)
    v = torch.zeros(2, 4, 128, dtype=torch.bfloat16, device=d)
    w = torch.ones(128, dtype=torch.float32, device=d)
    sk = torch.zeros(32, dtype=torch.float32, device=d)
    out = torch.zeros(2, 32, 128, dtype=torch.bfloat16, device=d)
    base = [q.data_ptr(), k.data_ptr(), v.data_ptr(), w.data_ptr(), w.data_ptr(), sk.data_ptr(), 0,
            cache.length.data_ptr(), 2, cache.k.data_ptr(), cache.vt.data_ptr(), cache.cap, 32, 4,
            128, 513, 1, 1.0e6, 1.0e-6, cache.workspace.data_ptr(), cache.workspace.numel(),
            out.data_ptr(), 0]
    assert fa.flint_attn_decode(*base) == fa.FLINT_OK
    torch.cuda.synchronize()
    for i, val, want in ((11, 520, fa.FLINT_ERR_SHAPE),       # cap not a multiple of 32
                         (11, 512, fa.FLINT_ERR_SHAPE),       # sliding ring smaller than the window
                         (12, 16, fa.FLINT_ERR_UNSUPPORTED),  # head layout
                         (15, -1, fa.FLINT_ERR_VALUE),        # window
                         (20, 64, fa.FLINT_ERR_WORKSPACE),
                         (0, 0, fa.FLINT_ERR_NULL),
                         (0, q.data_ptr() + 2, fa.FLINT_ERR_ALIGN)):
        bad = list(base)
        bad[i] = val
        assert fa.flint_attn_decode(*bad) == want, (i, val)


def test_long_full_context_batch():
    """8 sequences of 8192 cached tokens, the full layer (every key of every row checked)."""
    B, L = 8, 8192
    wl = make_custom(4008, [L + 1] * B, layers=(FULL,))
    _decode_and_check(wl, FULL, [L] * B, 1, L + 32, "full 8 x 8192")


def test_very_long_full_context():
    """One sequence with 131,071 cached tokens (the long-context prefill length)."""
    from oracle import flint_attention

    d = _d()
    L = 131071
    wl = make_long_decode(4009, L)
    k_all, v_all = wl.meta["k_all"], wl.meta["v_all"]
    cache = fa.KVCache(1, 0, max_tokens=L + 1, use_rope=False, device=d)
    kw = wl.k_norm_w.to(d)
    cache.append(k_all[:L].unsqueeze(0).contiguous().to(d), v_all[:L].unsqueeze(0).contiguous().to(d), kw)
    _log(f"[decode] full {L}: cache filled")
    out = cache.decode(wl.q.to(d), wl.k.to(d), wl.v.to(d), wl.q_norm_w.to(d), kw, wl.sinks.to(d))
    st, flags = cache.device_status()
    assert st == fa.FLINT_OK and flags == 0
    T = L + 1
    # only row T - 1 is computed, so the other query rows can be any values
    q_all = np.broadcast_to(f64(wl.q), (T, 32, 128))
    ref = flint_attention(q_all, f64(k_all), f64(v_all), f64(wl.q_norm_w), f64(wl.k_norm_w),
                          f64(wl.sinks), np.array([0, T]), window=0, use_rope=False, rows=[T - 1])
    vmax = float(np.max(np.abs(f64(v_all))))
    err = np.abs(to_np(out) - ref)
    _log(f"[decode] full {L}: max err {err.max() / vmax:.3e} x max|V|")
    assert err.max() <= 2e-2 * vmax and err.mean() <= 1e-3 * vmax


def test_decode_step_replayed_from_a_hip_graph():
    """One decode step (append, attention, merge: four launches) captured in a
    HIP graph. Every replay, with eager work and synchronizations between the
    replays, gives the eager step's output bit for bit (the step rewrites the
    same cache slot, so it is idempotent)."""
    d = _d()
    B, L = 4, 700
    rng = np.random.default_rng(31)
    bf = lambda *shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16).to(d)  # noqa: E731
    qw = torch.from_numpy((1 + 0.1 * rng.standard_normal(128)).astype(np.float32)).to(d)
    kw = torch.from_numpy((1 + 0.1 * rng.standard_normal(128)).astype(np.float32)).to(d)
    sinks = torch.from_numpy(rng.standard_normal(32).astype(np.float32)).to(d)
    cache = fa.KVCache(B, 0, max_tokens=L + 1, use_rope=False, device=d)
    cache.append(bf(B, L, 4, 128), bf(B, L, 4, 128), kw)
    q1, k1, v1 = bf(B, 32, 128), bf(B, 4, 128), bf(B, 4, 128)
    p = lambda t: int(t.data_ptr())  # noqa: E731

    def step(out, stream):
        return fa.flint_attn_decode(p(q1), p(k1), p(v1), p(qw), p(kw), p(sinks), 0, p(cache.length), B,
                                    p(cache.k), p(cache.vt), cache.cap, 32, 4, 128, 0, 0, 1.0e6, 1.0e-6,
                                    p(cache.workspace), cache.workspace.numel(), p(out),
                                    int(stream.cuda_stream))

    out_e = torch.empty(B, 32, 128, dtype=torch.bfloat16, device=d)
    assert step(out_e, torch.cuda.current_stream(d)) == 0
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert step(out_g, torch.cuda.current_stream(d)) == 0
    for i in range(4):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {i} differs from the eager step"
        float(torch.randn(1 << 20, device=d).sum())  # eager work between replays
    assert cache.device_status()[0] == fa.FLINT_OK


@pytest.mark.parametrize("layer", [FULL, SLIDING], ids=["full", "sliding"])
def test_decode_does_not_depend_on_workspace_contents(layer):
    """A decode step from identical caches gives the same bits on a zeroed
    workspace, on one filled with NaN bit patterns, and again on a zeroed one:
    the split partials and the merge read only what the step wrote."""
    wl = make_custom(341, [700, 300, 1500])
    prefix = [650, 250, 1400]
    d = _d()
    cu = i64(wl.cu_seqlens)
    rows = torch.as_tensor([int(cu[b]) + prefix[b] for b in range(3)])
    q, k, v = (wl.q[rows].contiguous().to(d), wl.k[rows].contiguous().to(d), wl.v[rows].contiguous().to(d))
    pos = None if wl.positions is None else wl.positions[rows].contiguous().to(d)
    qw, kw, sk = wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d)
    outs = []
    for fill in (0x00, 0xFF, 0x00):
        cache = _cache_for(wl, layer, prefix, 2048)
        cache.workspace.fill_(fill)
        out = cache.decode(q, k, v, qw, kw, sk, pos)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all(), f"fill {fill:#x}: non-finite output"
        outs.append((out.clone(), cache.k.clone(), cache.vt.clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_full_layer_wide_batch():
    """32 sequences (128 workgroups: the one-launch step also for caches longer
    than 1,024 slots) of mixed lengths at block edges, every step graded."""
    edges = [0, 1, 31, 32, 33, 255, 256, 257, 1000, 2049]
    prefix = [edges[i % len(edges)] + 7 * (i // len(edges)) for i in range(32)]
    steps = 2
    wl = make_custom(4010, [p + steps for p in prefix], layers=(FULL,))
    _decode_and_check(wl, FULL, prefix, steps, 2080, "full wide batch")


def test_full_cache_overflow_beside_a_valid_sequence():
    """Batch 2 over 2,048 slots (the split-K step): the full sequence reports
    the overflow and gets zeros, the other decodes normally."""
    d = _d()
    wl = make_custom(4011, [2049, 102], layers=(FULL,))
    cache = _cache_for(wl, FULL, [2048, 100], 2048)
    rows = np.array([2048, 2049 + 100])
    idx = torch.as_tensor(rows)
    out = cache.decode(wl.q[idx].contiguous().to(d), wl.k[idx].contiguous().to(d),
                       wl.v[idx].contiguous().to(d), wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d))
    st, flags = cache.device_status()
    assert st == fa.FLINT_ERR_DEVICE_DATA and flags & fa.FLINT_DEV_CACHE
    assert torch.count_nonzero(out[0]).item() == 0
    ref = oracle_for(wl, FULL, rows=rows[1:])
    grade(to_np(out[1:]), ref, wl, rows=rows[1:], what="valid sequence beside an overflow")
