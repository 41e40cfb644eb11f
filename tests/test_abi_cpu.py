"""C-ABI contract on the CPU: the library loads, exports every declared entry
point, and rejects bad arguments before touching the device."""

import ctypes
import os
import re
import subprocess

import pytest

import attention_head_rmsnorm_amd as fa
from attention_head_rmsnorm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint_attn.h")

FAKE = 1 << 20  # an aligned non-NULL address that is never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flint_(?:attn|proj)_\w+)\s*\(", text)))


def test_header_declares_binding_names():
    assert _declared() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (flint_(?:attn|proj)_\w+)", nm))
    assert set(_declared()) <= exported


def test_strerror_covers_every_status():
    seen = set()
    for st in range(0, -10, -1):
        msg = fa.flint_attn_strerror(st)
        assert msg and "unknown" not in msg
        seen.add(msg)
    assert len(seen) == 10
    assert "unknown" in fa.flint_attn_strerror(-99)


def test_fwd_kernel_query():
    k = fa.flint_attn_fwd_kernel
    assert k(0, 1) == 0
    assert k(-1, 1) == fa.FLINT_ERR_SHAPE and k(64, 0) == fa.FLINT_ERR_SHAPE
    # one 64-token sequence: 2 query blocks, far fewer than CUs -> the split kernel
    assert k(64, 1) == fa.FLINT_KERNEL_SPLIT
    # 8192 tokens: 256 query blocks per kv head -> the 8-wave kernel
    assert k(8192, 1) == fa.FLINT_KERNEL_WIDE
    # monotone in the number of query blocks
    seen_wide = False
    for T in range(32, 4096, 32):
        r = k(T, 1)
        assert r in (fa.FLINT_KERNEL_SPLIT, fa.FLINT_KERNEL_WIDE)
        if r == fa.FLINT_KERNEL_WIDE:
            seen_wide = True
        else:
            assert not seen_wide


def test_workspace_bytes_monotone_and_rejects_bad_sizes():
    ws = fa.flint_attn_workspace_bytes
    assert ws(-1, 1, 1) == 0 and ws(1, -1, 1) == 0 and ws(1, 1, -1) == 0
    assert ws(100, 1, 100, 8, 128) == 0 and ws(100, 1, 100, 4, 64) == 0
    prev = 0
    for T in (0, 1, 63, 64, 65, 1000, 8192, 131072):
        cur = ws(T, 1, T)
        assert cur >= prev
        prev = cur
    assert ws(8192, 2, 8192) >= ws(8192, 1, 8192)
    # the K/V tiles dominate: 2 KiB per token per kv head group pair, whole tiles
    assert ws(8192, 1, 8192) >= 4 * (8192 // 64 + 1) * 32768


# FLINT_MAX_SEQLEN of the header: the longest sequence the prefill kernels take
MAX_SEQLEN = int(re.search(r"#define FLINT_MAX_SEQLEN (\d+)", open(HEADER).read()).group(1))


def test_sequence_length_limit():
    assert MAX_SEQLEN == 1 << 21
    for ws in (fa.flint_attn_workspace_bytes, fa.flint_attn_f16_workspace_bytes,
               fa.flint_attn_bwd_workspace_bytes):
        assert ws(MAX_SEQLEN, 1, MAX_SEQLEN) > 0
        assert ws(MAX_SEQLEN, 1, MAX_SEQLEN + 1) == 0


def _call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, q_norm_w=FAKE, k_norm_w=FAKE, sink=FAKE, positions=0,
             cu_seqlens=FAKE, seqused=0, n_seqs=1, max_seqlen=64, total_tokens=64, num_q_heads=32,
             num_kv_heads=4, head_dim=128, window=513, use_rope=1, rope_theta=1e6, eps=1e-6,
             workspace=FAKE, workspace_bytes=0, out=FAKE, stream=0)
    a.update(over)
    return fa.flint_attn_fwd(**a)


@pytest.mark.parametrize("over,expect", [
    (dict(total_tokens=-1), fa.FLINT_ERR_SHAPE),
    (dict(n_seqs=-1), fa.FLINT_ERR_SHAPE),
    (dict(max_seqlen=-5), fa.FLINT_ERR_SHAPE),
    (dict(n_seqs=0), fa.FLINT_ERR_SHAPE),
    (dict(num_q_heads=16), fa.FLINT_ERR_UNSUPPORTED),
    (dict(num_kv_heads=8), fa.FLINT_ERR_UNSUPPORTED),
    (dict(head_dim=64), fa.FLINT_ERR_UNSUPPORTED),
    (dict(max_seqlen=MAX_SEQLEN + 1), fa.FLINT_ERR_UNSUPPORTED),
    (dict(window=-1), fa.FLINT_ERR_VALUE),
    (dict(eps=0.0), fa.FLINT_ERR_VALUE),
    (dict(eps=float("nan")), fa.FLINT_ERR_VALUE),
    (dict(rope_theta=0.0), fa.FLINT_ERR_VALUE),
    (dict(rope_theta=float("inf")), fa.FLINT_ERR_VALUE),
    (dict(q=0), fa.FLINT_ERR_NULL),
    (dict(k=0), fa.FLINT_ERR_NULL),
    (dict(v=0), fa.FLINT_ERR_NULL),
    (dict(q_norm_w=0), fa.FLINT_ERR_NULL),
    (dict(k_norm_w=0), fa.FLINT_ERR_NULL),
    (dict(sink=0), fa.FLINT_ERR_NULL),
    (dict(cu_seqlens=0), fa.FLINT_ERR_NULL),
    (dict(out=0), fa.FLINT_ERR_NULL),
    (dict(workspace=0), fa.FLINT_ERR_WORKSPACE),
    (dict(q=FAKE + 8), fa.FLINT_ERR_ALIGN),
    (dict(out=FAKE + 2), fa.FLINT_ERR_ALIGN),
    (dict(workspace=FAKE + 16), fa.FLINT_ERR_ALIGN),
    (dict(cu_seqlens=FAKE + 2), fa.FLINT_ERR_ALIGN),
    (dict(positions=FAKE + 1), fa.FLINT_ERR_ALIGN),
    (dict(workspace_bytes=1024), fa.FLINT_ERR_WORKSPACE),
])
def test_fwd_rejects_before_launch(over, expect):
    assert _call(**over) == expect


def test_fwd_nope_ignores_theta():
    # theta is unused on NoPE layers, so 0 is accepted there; the small
    # workspace is what is reported
    assert _call(use_rope=0, rope_theta=0.0, workspace_bytes=16) == fa.FLINT_ERR_WORKSPACE


def test_fwd_zero_tokens_is_a_no_op():
    # nothing is read or launched, so NULL pointers are fine
    assert _call(total_tokens=0, q=0, k=0, v=0, out=0, workspace=0, cu_seqlens=0) == fa.FLINT_OK


def test_mask_helper_validation():
    f = fa.flint_attn_seqused_from_mask
    assert f(FAKE, -1, 4, FAKE, FAKE, 0) == fa.FLINT_ERR_SHAPE
    assert f(0, 2, 4, FAKE, FAKE, 0) == fa.FLINT_ERR_NULL
    assert f(FAKE, 2, 4, 0, FAKE, 0) == fa.FLINT_ERR_NULL
    assert f(FAKE, 2, 4, FAKE + 2, FAKE, 0) == fa.FLINT_ERR_ALIGN


def test_device_status_validation():
    st, _ = fa.flint_attn_device_status(0, 0)
    assert st == fa.FLINT_ERR_NULL
    st, _ = fa.flint_attn_device_status(FAKE + 8, 0)
    assert st == fa.FLINT_ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(4, 32, 128, dtype=torch.bfloat16)
    k = torch.zeros(4, 4, 128, dtype=torch.bfloat16)
    w = torch.ones(128)
    with pytest.raises(ValueError):
        fa.flint_attn(q, k, k, w, w, torch.zeros(32))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library()


def test_c_struct_sizes():
    # int32 / float / size_t widths the ctypes declarations assume
    assert ctypes.sizeof(ctypes.c_size_t) == 8 and ctypes.sizeof(ctypes.c_void_p) == 8


def test_proj_validation():
    qkv = fa.flint_proj_qkv
    ok = dict(x=FAKE, w_q=FAKE, w_k=FAKE, w_v=FAKE, total_tokens=64, hidden=2048, num_q_heads=32,
              num_kv_heads=4, head_dim=128, q=FAKE, k=FAKE, v=FAKE, stream=0)

    def c(**over):
        a = dict(ok)
        a.update(over)
        return qkv(**a)
    assert c(total_tokens=-1) == fa.FLINT_ERR_SHAPE
    assert c(hidden=0) == fa.FLINT_ERR_SHAPE
    assert c(hidden=2050) == fa.FLINT_ERR_UNSUPPORTED and c(hidden=2080) == fa.FLINT_ERR_UNSUPPORTED
    assert c(num_kv_heads=8) == fa.FLINT_ERR_UNSUPPORTED
    assert c(x=0) == fa.FLINT_ERR_NULL and c(v=0) == fa.FLINT_ERR_NULL
    assert c(w_k=FAKE + 8) == fa.FLINT_ERR_ALIGN and c(q=FAKE + 2) == fa.FLINT_ERR_ALIGN
    assert c(total_tokens=0, x=0, q=0) == fa.FLINT_OK
    out = fa.flint_proj_out
    assert out(FAKE, FAKE, 64, 2000, 32, 128, FAKE, 0) == fa.FLINT_ERR_UNSUPPORTED
    assert out(FAKE, FAKE, 64, 2048, 16, 128, FAKE, 0) == fa.FLINT_ERR_UNSUPPORTED
    assert out(0, FAKE, 64, 2048, 32, 128, FAKE, 0) == fa.FLINT_ERR_NULL
    assert out(FAKE, FAKE, 64, 2048, 32, 128, FAKE + 4, 0) == fa.FLINT_ERR_ALIGN
    assert out(0, 0, 0, 2048, 32, 128, 0, 0) == fa.FLINT_OK


def test_bshd_plan_and_copy_validation():
    nb = fa.flint_attn_bshd_plan_bytes
    assert nb(-1, 4) == 0 and nb(2, 4) >= 4 * (8 + 6 * 8)
    plan = fa.flint_attn_bshd_plan
    assert plan(FAKE, FAKE, -1, 4, FAKE, 1 << 20, 0) == fa.FLINT_ERR_SHAPE
    assert plan(FAKE, FAKE, 1 << 16, 1 << 15, FAKE, 1 << 40, 0) == fa.FLINT_ERR_SHAPE
    assert plan(FAKE, FAKE, 2, 4, 0, 1 << 20, 0) == fa.FLINT_ERR_NULL
    assert plan(FAKE, FAKE + 2, 2, 4, FAKE, 1 << 20, 0) == fa.FLINT_ERR_ALIGN
    assert plan(FAKE, FAKE, 2, 4, FAKE, nb(2, 4) - 4, 0) == fa.FLINT_ERR_WORKSPACE
    cp = fa.flint_attn_copy_rows
    assert cp(FAKE, FAKE, -1, 16, 0, FAKE, 0) == fa.FLINT_ERR_SHAPE
    assert cp(FAKE, FAKE, 4, 6, 0, FAKE, 0) == fa.FLINT_ERR_SHAPE
    assert cp(0, FAKE, 4, 16, 0, FAKE, 0) == fa.FLINT_ERR_NULL
    assert cp(FAKE + 2, FAKE, 4, 16, 0, FAKE, 0) == fa.FLINT_ERR_ALIGN
    assert cp(0, 0, 0, 16, 0, 0, 0) == fa.FLINT_OK


def test_f16_workspace_adds_query_rows():
    a = fa.flint_attn_workspace_bytes(8192, 1, 8192)
    b = fa.flint_attn_f16_workspace_bytes(8192, 1, 8192)
    assert b >= a + 8192 * 32 * 128 * 2
    assert fa.flint_attn_f16_workspace_bytes(8192, 1, 8192, 8, 128) == 0
