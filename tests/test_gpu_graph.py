"""GPU: the forward and the backward under HIP graph capture.

Both entry points only enqueue kernels on the caller's stream: no allocation,
no synchronization and no memset nodes. So a caller can capture them in a
graph. Each test captures one call and replays it several times, with eager
work and synchronizations between the replays. Every replay must give the
eager call's outputs bit for bit: the kernels use no atomics in the values
they write, so a call is deterministic.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from workload import make_custom
from workload.gen import SLIDING, draw_dout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _p(t):
    return 0 if t is None else int(t.data_ptr())


def _replays(g, outs, refs):
    for i in range(3):
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"
        float(torch.randn(1 << 20, device=o.device).sum())  # eager work between replays


def _inputs(d):
    wl = make_custom(4242, [700, 130, 1, 257], layout="thd", seqused=[650, 130, 1, 200],
                     positions="random")
    t = dict(q=wl.q.to(d), k=wl.k.to(d), v=wl.v.to(d), qw=wl.q_norm_w.to(d), kw=wl.k_norm_w.to(d),
             sk=wl.sinks.to(d), pos=wl.positions.to(torch.int32).to(d), cu=wl.cu_seqlens.to(d),
             su=wl.seqused.to(d))
    return wl, t


def test_forward_replayed_from_a_hip_graph():
    d = torch.device("cuda", 0)
    wl, t = _inputs(d)
    T, n = wl.total_tokens, len(wl.cu_seqlens) - 1
    nbytes = fa.flint_attn_workspace_bytes(T, n, wl.max_seqlen)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=d)

    def call(out, stream):
        return fa.flint_attn_fwd(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["qw"]), _p(t["kw"]), _p(t["sk"]),
                                 _p(t["pos"]), _p(t["cu"]), _p(t["su"]), n, wl.max_seqlen, T, 32, 4, 128,
                                 SLIDING.window, 1, 1.0e6, 1.0e-6, _p(ws), nbytes, _p(out),
                                 int(stream.cuda_stream))

    ref = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=d)
    assert call(ref, torch.cuda.current_stream(d)) == fa.FLINT_OK
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert call(out, torch.cuda.current_stream(d)) == fa.FLINT_OK
    _replays(g, [out], [ref])


def test_backward_replayed_from_a_hip_graph():
    d = torch.device("cuda", 0)
    wl, t = _inputs(d)
    T, n = wl.total_tokens, len(wl.cu_seqlens) - 1
    o, lse = fa.flint_attn(t["q"], t["k"], t["v"], t["qw"], t["kw"], t["sk"], positions=t["pos"],
                           cu_seqlens=t["cu"], seqused=t["su"], max_seqlen=wl.max_seqlen,
                           window=SLIDING.window, use_rope=True, return_lse=True)
    dout = draw_dout(4242, T).to(d)
    nbytes = fa.flint_attn_bwd_workspace_bytes(T, n, wl.max_seqlen)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=d)

    def grads():
        return [torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]),
                torch.empty(128, dtype=torch.float32, device=d), torch.empty(128, dtype=torch.float32, device=d),
                torch.empty(32, dtype=torch.float32, device=d)]

    def call(gr, stream):
        return fa.flint_attn_bwd(_p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["qw"]), _p(t["kw"]), _p(t["sk"]),
                                 _p(t["pos"]), _p(t["cu"]), _p(t["su"]), n, wl.max_seqlen, T, 32, 4, 128,
                                 SLIDING.window, 1, 1.0e6, 1.0e-6, _p(o), _p(lse), _p(dout), _p(ws), nbytes,
                                 *[_p(x) for x in gr], int(stream.cuda_stream))

    ref = grads()
    assert call(ref, torch.cuda.current_stream(d)) == fa.FLINT_OK
    torch.cuda.synchronize()
    out = grads()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert call(out, torch.cuda.current_stream(d)) == fa.FLINT_OK
    _replays(g, out, ref)
    assert np.isfinite(ref[5].cpu().numpy()).all()


def _bshd_inputs(d):
    wl = make_custom(4343, [300, 300, 300], layout="bshd", seqused=[300, 120, 0])
    B, S = 3, 300
    t = dict(q=wl.q.to(d).view(B, S, 32, 128), k=wl.k.to(d).view(B, S, 4, 128),
             v=wl.v.to(d).view(B, S, 4, 128), qw=wl.q_norm_w.to(d), kw=wl.k_norm_w.to(d),
             sk=wl.sinks.to(d), mask=wl.attention_mask().to(d))
    return wl, t


def test_torch_wrapper_with_attention_mask_replayed_from_a_hip_graph():
    """flint_attn(..., attention_mask=..., sync=False) reads nothing back from
    the device, so the whole wrapper call (mask lengths, row starts, workspace
    and output allocation, the forward) can be captured; every replay equals
    the eager call, which equals the default (plan) path bit for bit."""
    d = torch.device("cuda", 0)
    wl, t = _bshd_inputs(d)
    kw = dict(attention_mask=t["mask"], window=SLIDING.window, use_rope=True)
    args = (t["q"], t["k"], t["v"], t["qw"], t["kw"], t["sk"])
    ref = fa.flint_attn(*args, sync=False, **kw)
    planned = fa.flint_attn(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ref, planned)
    s = torch.cuda.Stream(d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):  # warm the allocator's graph-capture path
        fa.flint_attn(*args, sync=False, **kw)
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fa.flint_attn(*args, sync=False, **kw)
    _replays(g, [out], [ref])


def test_unsynced_mask_with_a_hole_is_a_device_error():
    """Under sync=False a mask row with a hole becomes length -1: the forward
    reports FLINT_DEV_SEQUSED and leaves the output untouched; check=True
    raises it."""
    d = torch.device("cuda", 0)
    wl, t = _bshd_inputs(d)
    mask = t["mask"].clone()
    mask[1, 200] = 1  # row 1: 120 valid tokens, then a valid token after padding
    args = (t["q"], t["k"], t["v"], t["qw"], t["kw"], t["sk"])
    out = torch.full_like(t["q"], 3.0)
    nbytes = fa.flint_attn_workspace_bytes(900, 3, 300)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=d)
    fa.flint_attn(*args, attention_mask=mask, sync=False, out=out, workspace=ws)
    st, flags = fa.flint_attn_device_status(ws.data_ptr(), torch.cuda.current_stream(d).cuda_stream)
    assert st == fa.FLINT_ERR_DEVICE_DATA and flags & 16
    assert torch.all(out == 3.0)
    with pytest.raises(fa.FlintError):
        fa.flint_attn(*args, attention_mask=mask, sync=False, check=True)
    su = fa.seqused_from_mask(mask, check=False)
    assert su.tolist() == [300, -1, 0]
