"""Edge cases on the 8-wave attention kernel, and the streaming softmax in bf16.

Small problems run on the split 4-wave kernel (two workgroups per work item);
every workload of the benchmark runs on the 8-wave one. Each edge case here is
run on both: as it is, and with one extra 2048-token THD document packed
beside it, which raises the work-item count past the split kernel's limit.
THD documents are independent, so the original rows keep their exact values
and are graded against the oracle the same way; the test asserts which kernel
the forward launched (``flint_attn_fwd_kernel``).

The streaming path (running max seeded from the sink, lazy rescale) is taken
when the logit bound |q'| max|k'| or the sink exceeds 56 log2 units:
RMSNorm weights x2.2 (bound ~79) or sinks above +38.8 natural-log units.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from workload import Layer, make_custom, make_workload
from workload.gen import FULL, SLIDING

from .common import f64, oracle_for
from .rounding_bound import U_BF16, perturbation_sigma
from .gpu_common import (check_against_oracle, grade, huge_positions, kernel_of, run_gpu, to_np,
                         valid_rows, with_filler)
from .test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _both(wl):
    """(workload, rows, expected kernel) for the split and the 8-wave kernel."""
    T = wl.total_tokens
    rows = np.arange(T, dtype=np.int64)
    filled, frows = with_filler(wl)
    assert kernel_of(filled) == fa.FLINT_KERNEL_WIDE
    return [(wl, rows, kernel_of(wl)), (filled, frows, fa.FLINT_KERNEL_WIDE)]


# ----------------------------------------------------------------- the SMALL list on both kernels


@pytest.mark.parametrize("name,wl,layer", SMALL, ids=[c[0] for c in SMALL])
def test_small_on_wide_kernel(name, wl, layer):
    filled, rows = with_filler(wl)
    kern = kernel_of(filled)
    _log(f"[gpu] small case on the 8-wave kernel: {name} seed={wl.seed} T={filled.total_tokens} kernel={kern}")
    assert kern == fa.FLINT_KERNEL_WIDE
    stats, out = check_against_oracle(filled, layer, rows=rows)
    _log(f"      {stats}")


@pytest.mark.parametrize("name,wl,layer", SMALL, ids=[c[0] for c in SMALL])
def test_split_and_wide_kernels_agree(name, wl, layer):
    """The two kernels run the same per-tile steps in the same order: the
    original rows come out bit for bit equal."""
    filled, rows = with_filler(wl)
    a = run_gpu(wl, layer)
    b = run_gpu(filled, layer)
    torch.cuda.synchronize()
    _log(f"[gpu] split vs wide bitwise: {name} kernels {kernel_of(wl)} / {kernel_of(filled)}")
    assert torch.equal(a, b[: wl.total_tokens])


# ----------------------------------------------------------------- sinks, closed forms, invariances


def test_sink_minus_inf_both():
    for wl0 in (make_custom(220, [300, 45], layout="thd"),):
        for wl, rows, kern in _both(wl0):
            assert kernel_of(wl) == kern
            for layer in (SLIDING, FULL):
                _log(f"[gpu] sink -inf kernel={kern} {layer.name}")
                check_against_oracle(wl, layer, rows=rows, sinks=np.full(32, -np.inf, np.float32))


def test_sink_large_gives_zero_output_both():
    for wl, rows, kern in _both(make_custom(221, [200])):
        out = run_gpu(wl, SLIDING, sinks=np.full(32, 80.0, np.float32))
        torch.cuda.synchronize()
        _log(f"[gpu] sink +80 kernel={kern}")
        assert float(out[: len(rows)].float().abs().max()) < 1e-20


def test_mixed_sinks_both():
    s = np.random.default_rng(0).normal(0, 3, 32).astype(np.float32)
    s[::5] = -np.inf
    s[1] = 12.0
    for wl, rows, kern in _both(make_custom(222, [170, 3, 90], layout="thd")):
        for layer in (SLIDING, FULL):
            _log(f"[gpu] mixed sinks kernel={kern} {layer.name}")
            check_against_oracle(wl, layer, rows=rows, sinks=s)


def test_zero_query_closed_form_wide():
    """q = 0 makes every allowed logit 0: O[t] = sum_A v / (e^sink + |A|),
    here on the 8-wave kernel (a 2048-token sequence)."""
    wl = make_custom(223, [2048], q_scale=0.0)
    assert kernel_of(wl) == fa.FLINT_KERNEL_WIDE
    v = f64(wl.v)
    s = f64(wl.sinks)
    cs = np.concatenate([np.zeros((1, 4, 128)), np.cumsum(v, 0)], 0)
    for layer in (SLIDING, FULL):
        out = to_np(run_gpu(wl, layer))
        t = np.arange(2048)
        lo = np.zeros(2048, np.int64) if layer.window == 0 else np.maximum(0, t - layer.window + 1)
        vs = cs[t + 1] - cs[lo]                      # [T, 4, 128]
        n = (t + 1 - lo).astype(np.float64)           # [T]
        g = np.arange(32) // 8
        ref = vs[:, g, :] / (np.exp(s)[None, :, None] + n[:, None, None])
        grade(out, ref, wl, what=f"q=0 wide {layer.name}")


def test_nope_ignores_positions_bitwise_wide():
    wl = make_custom(224, [400, 100, 2048], layout="thd")
    assert kernel_of(wl) == fa.FLINT_KERNEL_WIDE
    a = run_gpu(wl, FULL)
    b = run_gpu(wl, FULL, positions=np.random.default_rng(3).integers(0, 262144, wl.total_tokens))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_thd_document_equals_alone_bitwise_wide():
    """Each document of a packing equals the document run alone, with every
    run on the 8-wave kernel (a 2048-token document sits in each packing)."""
    lengths = [300, 77, 513, 2048]
    wl = make_custom(225, lengths, layout="thd")
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for layer in (SLIDING, FULL):
        packed = run_gpu(wl, layer)
        for d, n in enumerate(lengths[:3]):
            a, b = int(cu[d]), int(cu[d + 1])
            # document d alone, beside the same 2048-token document
            f = cu[3]
            idx = torch.cat([torch.arange(a, b), torch.arange(int(f), int(f) + 2048)])
            one = make_custom(225, [n, 2048], layout="thd")
            one.q, one.k, one.v = wl.q[idx].clone(), wl.k[idx].clone(), wl.v[idx].clone()
            one.positions = wl.positions[idx].clone()
            one.q_norm_w, one.k_norm_w, one.sinks = wl.q_norm_w, wl.k_norm_w, wl.sinks
            assert kernel_of(one) == fa.FLINT_KERNEL_WIDE
            alone = run_gpu(one, layer)
            torch.cuda.synchronize()
            assert torch.equal(packed[a:b], alone[:n]), f"document {d} {layer.name}"


@pytest.mark.parametrize("layer", [SLIDING, Layer(window=0, use_rope=True)], ids=["sliding", "full-rope"])
def test_positions_beyond_2_24_both_kernels(layer):
    """RoPE positions up to the int32 limits, beside small ones in the same
    waves: keys (the K tiles) and queries (the prologue) graded against the
    oracle, which turns them in FP64, on both kernels."""
    wl = huge_positions(make_custom(241, [300, 77, 150], layout="thd"))
    for w, rows, kern in _both(wl):
        _log(f"[gpu] positions beyond 2^24: {layer.name} T={w.total_tokens} kernel={kern}")
        assert kernel_of(w) == kern
        stats, _ = check_against_oracle(w, layer, rows=rows)
        _log(f"      {stats}")


def test_deterministic_bitwise_wide():
    wl = make_custom(226, [900, 50, 2048], layout="thd")
    for layer in (SLIDING, FULL):
        a = run_gpu(wl, layer)
        b = run_gpu(wl, layer)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_output_guard_bands_untouched_wide():
    wl = make_custom(228, [257, 31, 2048], layout="thd")
    T = wl.total_tokens
    buf = torch.full(((T + 2) * 32 * 128,), 12345.0, dtype=torch.bfloat16, device="cuda")
    out = buf[32 * 128:(T + 1) * 32 * 128].view(T, 32, 128)
    run_gpu(wl, SLIDING, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:32 * 128] == 12345.0) and torch.all(buf[(T + 1) * 32 * 128:] == 12345.0)


def test_workspace_reuse_and_stale_content_wide():
    wl1 = make_custom(229, [3000], layout="thd")
    wl2 = make_custom(230, [64, 700, 2048], layout="thd")
    nbytes = fa.flint_attn_workspace_bytes(3000, 3, 3000)
    ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    r1 = run_gpu(wl2, SLIDING)
    run_gpu(wl1, FULL, workspace=ws)
    r2 = run_gpu(wl2, SLIDING, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)


# ----------------------------------------------------------------- the streaming branch in bf16


@pytest.mark.parametrize("scale", [1.6, 2.2])
def test_large_logits_both_kernels(scale):
    """x1.6 stays on the unshifted path (bound ~41 log2 units), x2.2 (~79)
    takes the streaming path, on both kernels."""
    wl0 = make_custom(240 + int(scale * 10), [700, 130], layout="thd", norm_scale=scale)
    for wl, rows, kern in _both(wl0):
        for layer in (SLIDING, FULL):
            _log(f"[gpu] norm weights x{scale} kernel={kern} {layer.name}")
            stats, _ = check_against_oracle(wl, layer, rows=rows)
            _log(f"      {stats}")
            check_against_oracle(wl, layer, rows=rows, sinks=np.full(32, -np.inf, np.float32))


def test_streaming_large_sinks_both_kernels():
    """Sinks of +40 to +55 natural-log units (58-79 in log2 units, past the
    unshifted bound) beside logits of the same size (weights x2.2): the sink
    is the running max for many rows, and keys overtake it in others."""
    s = np.random.default_rng(7).uniform(40.0, 55.0, 32).astype(np.float32)
    wl0 = make_custom(250, [700, 130], layout="thd", norm_scale=2.2)
    for wl, rows, kern in _both(wl0):
        for layer in (SLIDING, FULL):
            ref = oracle_for(wl, layer, rows=rows, sinks=s.astype(np.float64), debug=True)[1]
            ps = ref["p_sink"][valid_rows(wl)[rows]]
            _log(f"[gpu] sinks +40..+55 kernel={kern} {layer.name}: p_sink in "
                 f"[{ps.min():.3g}, {ps.max():.3g}], median {np.median(ps):.3g}")
            stats, _ = check_against_oracle(wl, layer, rows=rows, sinks=s)
            _log(f"      {stats}")


def test_streaming_sink_plus40_unit_weights():
    """A sink of +40 (57.7 log2 units) alone puts every wave on the streaming
    path with ordinary weights; the output is tiny and must still match."""
    s = np.full(32, 40.0, np.float32)
    for wl, rows, kern in _both(make_custom(251, [600, 90], layout="thd")):
        for layer in (SLIDING, FULL):
            check_against_oracle(wl, layer, rows=rows, sinks=s)


@pytest.mark.parametrize("sink", [-1.0e6, -1.0e9])
def test_streaming_very_negative_sink(sink):
    """A finite sink far below every logit on the streaming path (x2.2
    weights): the sink's weight underflows to 0 and the rows are plain softmax
    attention, as with sink = -inf, on both kernels."""
    s = np.full(32, sink, np.float32)
    s[3] = 0.5  # one ordinary head beside them
    wl0 = make_custom(252, [700, 130], layout="thd", norm_scale=2.2)
    for wl, rows, kern in _both(wl0):
        for layer in (SLIDING, FULL):
            _log(f"[gpu] sink {sink:g} kernel={kern} {layer.name}")
            stats, _ = check_against_oracle(wl, layer, rows=rows, sinks=s)
            _log(f"      {stats}")
            a = run_gpu(wl, layer, sinks=s)
            b = run_gpu(wl, layer, sinks=np.where(np.arange(32) == 3, 0.5, -np.inf).astype(np.float32))
            torch.cuda.synchronize()
            got, inf_ref = to_np(a[: len(rows)]), to_np(b[: len(rows)])
            vmax = float(np.abs(f64(wl.v)).max())
            assert np.abs(got - inf_ref).max() <= 1e-2 * vmax


# ----------------------------------------------------------------- x3 weights: a derived bound

def test_weights_x3_within_rounding_bound():
    """RMSNorm weights x3 (logits up to ~100 natural-log units, near one-hot
    rows, streaming path): the error is graded per element against the
    first-order effect of the bf16 roundings, |err| <= 6 sigma + 2^-8 |O| +
    1e-3 max|V| (sigma from perturbation_sigma, the output's own bf16
    rounding, and slack for FP32 accumulation), and on average
    mean|err| <= mean(sigma) + 1e-3 max|V|."""
    wl0 = make_custom(253, [700, 130], layout="thd", norm_scale=3.0)
    rows0 = np.unique(np.concatenate([np.arange(0, 830, 7), [0, 1, 2, 512, 513, 699, 700, 829]]))
    for wl, _, kern in _both(wl0):
        for layer in (SLIDING, FULL):
            got = to_np(run_gpu(wl, layer)[torch.as_tensor(rows0, device="cuda")])
            sig, ref = perturbation_sigma(wl, layer, rows0)
            vmax = float(np.abs(f64(wl.v)).max())
            err = np.abs(got - ref)
            bound = 6.0 * sig + U_BF16 * np.abs(ref) + 1e-3 * vmax
            worst = float((err / bound).max())
            _log(f"[gpu] weights x3 kernel={kern} {layer.name}: max err {err.max():.3g} "
                 f"(plain bar {2e-2 * vmax:.3g}), max err/bound {worst:.3f}, "
                 f"mean err {err.mean():.3g} vs mean sigma {sig.mean():.3g}")
            assert np.all(np.isfinite(got))
            assert worst <= 1.0
            assert err.mean() <= sig.mean() + 1e-3 * vmax
