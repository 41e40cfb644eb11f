"""flint_attn_fwd_static (no allocation, static per-GPU scratch) against
flint_attn_fwd: the same kernels on the same inputs give the same bits, on two
calls in a row (the second smaller, on scratch the first one left behind),
and sizes beyond the scratch are refused before any launch."""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from workload import make_custom, make_workload
from workload.gen import FULL, SLIDING

from .gpu_common import grade, to_np
from .common import oracle_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _args(wl, layer, dev):
    t = dict(q=wl.q.to(dev), k=wl.k.to(dev), v=wl.v.to(dev), qw=wl.q_norm_w.to(dev),
             kw=wl.k_norm_w.to(dev), sk=wl.sinks.to(dev), cu=wl.cu_seqlens.to(dev),
             su=None if wl.seqused is None else wl.seqused.to(dev),
             pos=None if wl.positions is None else wl.positions.to(dev))
    p = lambda x: 0 if x is None else int(x.data_ptr())  # noqa: E731
    head = [p(t["q"]), p(t["k"]), p(t["v"]), p(t["qw"]), p(t["kw"]), p(t["sk"]), p(t["pos"]),
            p(t["cu"]), p(t["su"]), wl.n_seqs, wl.max_seqlen, wl.total_tokens, 32, 4, 128,
            layer.window, int(layer.use_rope), layer.theta, layer.eps]
    return t, head


def _both(wl, layer):
    dev = torch.device("cuda", 0)
    keep, head = _args(wl, layer, dev)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    T = wl.total_tokens
    ref = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=dev)
    got = torch.full((T, 32, 128), 7.0, dtype=torch.bfloat16, device=dev)
    nbytes = fa.flint_attn_workspace_bytes(T, wl.n_seqs, wl.max_seqlen)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = fa.flint_attn_fwd(*head, int(ws.data_ptr()), nbytes, int(ref.data_ptr()), sh)
    assert st == fa.FLINT_OK, fa.flint_attn_strerror(st)
    st = fa.flint_attn_fwd_static(*head, int(got.data_ptr()), sh)
    assert st == fa.FLINT_OK, fa.flint_attn_strerror(st)
    torch.cuda.synchronize()
    del keep
    return got, ref


def test_static_scratch_matches_workspace_entry_point_twice():
    """A large call (full NoPE, S=8192) then a smaller ragged one (sliding
    RoPE, THD) on the scratch the first call filled: both equal the
    workspace entry point bit for bit, and the smaller one also meets the
    oracle bar."""
    wl1 = make_workload("tstar")
    print(f"[gpu] static scratch call 1: T={wl1.total_tokens} full NoPE", flush=True)
    g1, r1 = _both(wl1, FULL)
    assert torch.equal(g1, r1)
    wl2 = make_custom(301, [700, 33, 1500], layout="thd")
    print(f"[gpu] static scratch call 2: T={wl2.total_tokens} sliding RoPE THD", flush=True)
    g2, r2 = _both(wl2, SLIDING)
    assert torch.equal(g2, r2)
    grade(to_np(g2), oracle_for(wl2, SLIDING), wl2, what="static scratch, second call")


def test_static_scratch_refuses_oversize():
    """Sizes whose workspace exceeds the scratch return FLINT_ERR_TOO_LARGE and
    leave the output untouched."""
    dev = torch.device("cuda", 0)
    T = 1 << 16  # 64K tokens in one sequence need ~130 MiB of tiles
    assert fa.flint_attn_workspace_bytes(T, 1, T) > fa.FLINT_ATTN_STATIC_SCRATCH_BYTES
    out = torch.full((4,), 3.0, dtype=torch.bfloat16, device=dev)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    st = fa.flint_attn_fwd_static(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 0, 1 << 20, 0,
                                  1, T, T, 32, 4, 128, 0, 0, 1.0e6, 1.0e-6, int(out.data_ptr()), sh)
    assert st == fa.FLINT_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
