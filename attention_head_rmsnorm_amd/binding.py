"""ctypes binding of libflint_attn.so.

The functions named like the C entry points (``flint_attn_fwd`` and friends)
take the same arguments as the C ABI: device pointers as ints, sizes and a
stream handle. ``flint_attn`` is a convenience layer over them for torch
tensors: it checks dtypes and layouts, allocates the output and the workspace
with torch, and passes torch's current stream. Every step of the computation
runs in the library's HIP kernels; nothing here computes any part of the layer.
There is no fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes

import numpy as np
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflint_attn.so")

NUM_Q_HEADS = 32
NUM_KV_HEADS = 4
HEAD_DIM = 128

FLINT_OK = 0
FLINT_ERR_NULL = -1
FLINT_ERR_SHAPE = -2
FLINT_ERR_UNSUPPORTED = -3
FLINT_ERR_VALUE = -4
FLINT_ERR_WORKSPACE = -5
FLINT_ERR_ALIGN = -6
FLINT_ERR_HIP = -7
FLINT_ERR_DEVICE_DATA = -8
FLINT_ERR_TOO_LARGE = -9
FLINT_ATTN_STATIC_SCRATCH_BYTES = 64 << 20

FLINT_DEV_CACHE = 32

FLINT_PHASE_SCHEDULE = 1
FLINT_PHASE_KV = 2
FLINT_PHASE_ATTEND = 4
FLINT_PHASE_ALL = 7

FLINT_KERNEL_WIDE = 1   # one 8-wave workgroup per work item
FLINT_KERNEL_SPLIT = 2  # two 4-wave workgroups per work item (small problems)

EXPORTED = (
    "flint_attn_workspace_bytes",
    "flint_attn_fwd",
    "flint_attn_fwd_phases",
    "flint_attn_seqused_from_mask",
    "flint_attn_device_status",
    "flint_attn_strerror",
    "flint_attn_decode_workspace_bytes",
    "flint_attn_kv_append",
    "flint_attn_decode",
    "flint_attn_fwd_lse",
    "flint_attn_bwd_workspace_bytes",
    "flint_attn_bwd",
    "flint_attn_f16_workspace_bytes",
    "flint_attn_fwd_f16",
    "flint_attn_bshd_plan_bytes",
    "flint_attn_bshd_plan",
    "flint_attn_copy_rows",
    "flint_proj_qkv",
    "flint_proj_out",
    "flint_attn_fwd_kernel",
    "flint_attn_fwd_static",
)

_lib: Optional[ctypes.CDLL] = None


class FlintError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = flint_attn_strerror(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Loads the in-tree HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m attention_head_rmsnorm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.flint_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.flint_attn_workspace_bytes.restype = sz
    lib.flint_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i32, i32, f32, f32, vp, sz, vp, vp]
    lib.flint_attn_fwd.restype = ctypes.c_int
    lib.flint_attn_fwd_phases.argtypes = lib.flint_attn_fwd.argtypes + [i32]
    lib.flint_attn_fwd_phases.restype = ctypes.c_int
    lib.flint_attn_seqused_from_mask.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.flint_attn_seqused_from_mask.restype = ctypes.c_int
    lib.flint_attn_device_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.flint_attn_device_status.restype = ctypes.c_int
    lib.flint_attn_strerror.argtypes = [ctypes.c_int]
    lib.flint_attn_strerror.restype = ctypes.c_char_p
    lib.flint_attn_decode_workspace_bytes.argtypes = [i32, i32]
    lib.flint_attn_decode_workspace_bytes.restype = sz
    lib.flint_attn_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32,
                                         i32, f32, f32, vp, sz, vp]
    lib.flint_attn_kv_append.restype = ctypes.c_int
    lib.flint_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                      i32, i32, i32, f32, f32, vp, sz, vp, vp]
    lib.flint_attn_decode.restype = ctypes.c_int
    lib.flint_attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       i32, i32, i32, f32, f32, vp, sz, vp, vp, vp]
    lib.flint_attn_fwd_lse.restype = ctypes.c_int
    lib.flint_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.flint_attn_bwd_workspace_bytes.restype = sz
    lib.flint_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   i32, i32, f32, f32, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp]
    lib.flint_attn_bwd.restype = ctypes.c_int
    lib.flint_attn_f16_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.flint_attn_f16_workspace_bytes.restype = sz
    lib.flint_attn_fwd_f16.argtypes = lib.flint_attn_fwd.argtypes
    lib.flint_attn_fwd_f16.restype = ctypes.c_int
    lib.flint_attn_bshd_plan_bytes.argtypes = [i32, i32]
    lib.flint_attn_bshd_plan_bytes.restype = sz
    lib.flint_attn_bshd_plan.argtypes = [vp, vp, i32, i32, vp, sz, vp]
    lib.flint_attn_bshd_plan.restype = ctypes.c_int
    lib.flint_attn_copy_rows.argtypes = [vp, vp, i32, i32, ctypes.c_uint32, vp, vp]
    lib.flint_attn_copy_rows.restype = ctypes.c_int
    lib.flint_proj_qkv.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.flint_proj_qkv.restype = ctypes.c_int
    lib.flint_proj_out.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
    lib.flint_proj_out.restype = ctypes.c_int
    lib.flint_attn_fwd_kernel.argtypes = [i32, i32]
    lib.flint_attn_fwd_kernel.restype = ctypes.c_int
    lib.flint_attn_fwd_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          i32, i32, i32, ctypes.c_float, ctypes.c_float, vp, vp]
    lib.flint_attn_fwd_static.restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------------- raw C ABI


def flint_attn_workspace_bytes(total_tokens: int, n_seqs: int, max_seqlen: int,
                               num_kv_heads: int = NUM_KV_HEADS, head_dim: int = HEAD_DIM) -> int:
    return int(load_library().flint_attn_workspace_bytes(total_tokens, n_seqs, max_seqlen,
                                                         num_kv_heads, head_dim))


def flint_attn_fwd(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                   max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                   rope_theta, eps, workspace, workspace_bytes, out, stream) -> int:
    """The C entry point with pointer arguments as ints (0 = NULL); returns the status."""
    return int(load_library().flint_attn_fwd(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                             cu_seqlens, seqused, n_seqs, max_seqlen,
                                             total_tokens, num_q_heads, num_kv_heads, head_dim,
                                             window, use_rope, rope_theta, eps, workspace,
                                             workspace_bytes, out, stream))


def flint_attn_fwd_phases(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused,
                          n_seqs, max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim,
                          window, use_rope, rope_theta, eps, workspace, workspace_bytes, out,
                          stream, phases) -> int:
    """flint_attn_fwd restricted to the FLINT_PHASE_* bits in ``phases``; returns the status."""
    return int(load_library().flint_attn_fwd_phases(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                                    cu_seqlens, seqused, n_seqs, max_seqlen,
                                                    total_tokens, num_q_heads, num_kv_heads,
                                                    head_dim, window, use_rope, rope_theta, eps,
                                                    workspace, workspace_bytes, out, stream,
                                                    phases))


def flint_attn_fwd_lse(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                       max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window,
                       use_rope, rope_theta, eps, workspace, workspace_bytes, out, lse,
                       stream) -> int:
    """flint_attn_fwd that also writes the per-row normalizer lse (float32 [T, 32])."""
    return int(load_library().flint_attn_fwd_lse(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                                 cu_seqlens, seqused, n_seqs, max_seqlen,
                                                 total_tokens, num_q_heads, num_kv_heads,
                                                 head_dim, window, use_rope, rope_theta, eps,
                                                 workspace, workspace_bytes, out, lse, stream))


def flint_attn_f16_workspace_bytes(total_tokens: int, n_seqs: int, max_seqlen: int,
                                   num_kv_heads: int = NUM_KV_HEADS,
                                   head_dim: int = HEAD_DIM) -> int:
    return int(load_library().flint_attn_f16_workspace_bytes(total_tokens, n_seqs, max_seqlen,
                                                             num_kv_heads, head_dim))


def flint_attn_fwd_f16(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                       max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window,
                       use_rope, rope_theta, eps, workspace, workspace_bytes, out, stream) -> int:
    """The FP16 attention-compute variant (FP32 q, k, v and out); returns the status."""
    return int(load_library().flint_attn_fwd_f16(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                                 cu_seqlens, seqused, n_seqs, max_seqlen,
                                                 total_tokens, num_q_heads, num_kv_heads,
                                                 head_dim, window, use_rope, rope_theta, eps,
                                                 workspace, workspace_bytes, out, stream))


def flint_attn_bshd_plan_bytes(batch: int, seqlen: int) -> int:
    return int(load_library().flint_attn_bshd_plan_bytes(batch, seqlen))


def flint_attn_bshd_plan(attention_mask, document_ids, batch, seqlen, plan, plan_bytes,
                         stream) -> int:
    """THD description of BSHD input with a mask and/or document ids; returns the status."""
    return int(load_library().flint_attn_bshd_plan(attention_mask, document_ids, batch, seqlen,
                                                   plan, plan_bytes, stream))


def flint_attn_copy_rows(src, index, n_rows, row_bytes, fill, dst, stream) -> int:
    """dst row r = src row index[r] (fill words where index[r] < 0); returns the status."""
    return int(load_library().flint_attn_copy_rows(src, index, n_rows, row_bytes, fill, dst,
                                                   stream))


def flint_proj_qkv(x, w_q, w_k, w_v, total_tokens, hidden, num_q_heads, num_kv_heads, head_dim,
                   q, k, v, stream) -> int:
    """q, k, v projections of the hidden states in one launch; returns the status."""
    return int(load_library().flint_proj_qkv(x, w_q, w_k, w_v, total_tokens, hidden, num_q_heads,
                                             num_kv_heads, head_dim, q, k, v, stream))


def flint_proj_out(o, w_o, total_tokens, hidden, num_q_heads, head_dim, y, stream) -> int:
    """Output projection of the layer's output; returns the status."""
    return int(load_library().flint_proj_out(o, w_o, total_tokens, hidden, num_q_heads, head_dim,
                                             y, stream))


def flint_attn_bwd_workspace_bytes(total_tokens: int, n_seqs: int, max_seqlen: int,
                                   num_kv_heads: int = NUM_KV_HEADS,
                                   head_dim: int = HEAD_DIM) -> int:
    return int(load_library().flint_attn_bwd_workspace_bytes(total_tokens, n_seqs, max_seqlen,
                                                             num_kv_heads, head_dim))


def flint_attn_bwd(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                   max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                   rope_theta, eps, out, lse, dout, workspace, workspace_bytes, dq, dk, dv,
                   dq_norm_w, dk_norm_w, dsink, stream) -> int:
    """The backward C entry point with pointer arguments as ints; returns the status."""
    return int(load_library().flint_attn_bwd(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                             cu_seqlens, seqused, n_seqs, max_seqlen,
                                             total_tokens, num_q_heads, num_kv_heads, head_dim,
                                             window, use_rope, rope_theta, eps, out, lse, dout,
                                             workspace, workspace_bytes, dq, dk, dv, dq_norm_w,
                                             dk_norm_w, dsink, stream))


def flint_attn_seqused_from_mask(mask, batch, seqlen, seqused, n_bad, stream) -> int:
    return int(load_library().flint_attn_seqused_from_mask(mask, batch, seqlen, seqused, n_bad,
                                                           stream))


def flint_attn_device_status(workspace, stream):
    """Returns (status, flags) after synchronizing the stream."""
    flags = ctypes.c_int32(0)
    st = int(load_library().flint_attn_device_status(workspace, stream, ctypes.byref(flags)))
    return st, int(flags.value)


def flint_attn_fwd_static(q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs,
                          max_seqlen, total_tokens, num_q_heads, num_kv_heads, head_dim, window,
                          use_rope, rope_theta, eps, out, stream) -> int:
    """flint_attn_fwd with the library's static per-GPU scratch as workspace
    (no allocation; FLINT_ERR_TOO_LARGE beyond FLINT_ATTN_STATIC_SCRATCH_BYTES)."""
    return int(load_library().flint_attn_fwd_static(
        q, k, v, q_norm_w, k_norm_w, sink, positions, cu_seqlens, seqused, n_seqs, max_seqlen,
        total_tokens, num_q_heads, num_kv_heads, head_dim, window, use_rope, rope_theta, eps, out,
        stream))


def flint_attn_fwd_kernel(total_tokens: int, n_seqs: int) -> int:
    """FLINT_KERNEL_WIDE or FLINT_KERNEL_SPLIT: the attention kernel a bf16
    forward of these sizes launches (0 for no tokens, negative on bad sizes)."""
    return int(load_library().flint_attn_fwd_kernel(total_tokens, n_seqs))


def flint_attn_strerror(status: int) -> str:
    return load_library().flint_attn_strerror(int(status)).decode()


def flint_attn_decode_workspace_bytes(batch: int, cache_cap: int) -> int:
    return int(load_library().flint_attn_decode_workspace_bytes(batch, cache_cap))


def flint_attn_kv_append(k, v, k_norm_w, positions, cache_len, batch, n_new, k_cache, vt_cache,
                         cache_cap, num_kv_heads, head_dim, window, use_rope, rope_theta, eps,
                         workspace, workspace_bytes, stream) -> int:
    """The C entry point with pointer arguments as ints (0 = NULL); returns the status."""
    return int(load_library().flint_attn_kv_append(k, v, k_norm_w, positions, cache_len, batch,
                                                   n_new, k_cache, vt_cache, cache_cap,
                                                   num_kv_heads, head_dim, window, use_rope,
                                                   rope_theta, eps, workspace, workspace_bytes,
                                                   stream))


def flint_attn_decode(q, k, v, q_norm_w, k_norm_w, sink, positions, cache_len, batch, k_cache,
                      vt_cache, cache_cap, num_q_heads, num_kv_heads, head_dim, window, use_rope,
                      rope_theta, eps, workspace, workspace_bytes, out, stream) -> int:
    """The C entry point with pointer arguments as ints (0 = NULL); returns the status."""
    return int(load_library().flint_attn_decode(q, k, v, q_norm_w, k_norm_w, sink, positions,
                                                cache_len, batch, k_cache, vt_cache, cache_cap,
                                                num_q_heads, num_kv_heads, head_dim, window,
                                                use_rope, rope_theta, eps, workspace,
                                                workspace_bytes, out, stream))


# ----------------------------------------------------------------- torch layer


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(device) -> int:
    import torch

    return int(torch.cuda.current_stream(device).cuda_stream)


def seqused_from_mask(attention_mask, check: bool = True):
    """[B, S] binary mask (1 = valid, trailing padding only) -> int32 [B] on the device.

    With ``check`` the host reads the count of rows that are not trailing
    padding and raises if there is one (a synchronization); without it such
    rows get length -1, which the forward reports as a device-data error."""
    import torch

    if attention_mask.dim() != 2:
        raise ValueError("attention_mask must be [batch, seqlen]")
    m = attention_mask
    if m.dtype != torch.uint8:
        m = (m != 0).to(torch.uint8)
    m = m.contiguous()
    B, S = m.shape
    seqused = torch.empty(B, dtype=torch.int32, device=m.device)
    n_bad = torch.empty(1, dtype=torch.int32, device=m.device)
    st = flint_attn_seqused_from_mask(_ptr(m), B, S, _ptr(seqused), _ptr(n_bad),
                                      _stream_handle(m.device))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_seqused_from_mask")
    if check and int(n_bad.item()) != 0:
        raise ValueError("attention_mask has non-trailing padding; arbitrary padding uses THD "
                         "packing (pass cu_seqlens)")
    return seqused


class _Args:
    """The THD description of a call: T tokens in n sequences (cu, seqused,
    positions); for packed BSHD input also `pack` (source row of each stream
    token) and `unpack` (stream token of each source row, -1 on padding)."""

    def __init__(self, T, n, mx, cu, seqused, positions, pack=None, unpack=None):
        self.T, self.n, self.mx = T, n, mx
        self.cu, self.seqused, self.positions = cu, seqused, positions
        self.pack, self.unpack = pack, unpack

    def gather(self, t):
        """Rows of t (leading dims flattened) in stream order (t itself when not packed)."""
        import torch

        if self.pack is None:
            return t
        rows = t.reshape(self.unpack.numel(), -1)
        dst = torch.empty((self.T,) + tuple(t.shape[2:]), dtype=t.dtype, device=t.device)
        _copy_rows(rows, self.pack, self.T, dst)
        return dst

    def scatter(self, packed, out, fill=0):
        """Stream-order rows back to out's rows, `fill` (a 32-bit word) on padding."""
        if self.pack is not None:
            _copy_rows(packed.reshape(self.T, -1), self.unpack, self.unpack.numel(), out, fill)
        return out


def _copy_rows(src, index, n_rows, dst, fill=0):
    """dst (n_rows rows) row r = src row index[r], `fill` words where index[r] < 0."""
    if n_rows == 0:
        return
    row_bytes = dst.numel() * dst.element_size() // n_rows
    st = flint_attn_copy_rows(_ptr(src), _ptr(index), n_rows, row_bytes, fill, _ptr(dst),
                              _stream_handle(dst.device))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_copy_rows")


def bshd_plan(attention_mask, document_ids, batch: int, seqlen: int, device):
    """Runs the plan kernel and reads its counts (one host synchronization).

    Returns (info, cu, seqused, pack, unpack): info = (n_seqs, max_seqlen,
    total_tokens, packed, valid tokens, documents); the rest are views of the
    plan on the device."""
    import torch

    m = None
    if attention_mask is not None:
        if tuple(attention_mask.shape) != (batch, seqlen):
            raise ValueError("attention_mask must be [batch, seqlen]")
        m = attention_mask if attention_mask.dtype == torch.uint8 else (attention_mask != 0).to(torch.uint8)
        m = m.contiguous()
    d = None
    if document_ids is not None:
        if tuple(document_ids.shape) != (batch, seqlen):
            raise ValueError("document_ids must be [batch, seqlen]")
        d = document_ids.to(torch.int32).contiguous()
    N = batch * seqlen
    nbytes = flint_attn_bshd_plan_bytes(batch, seqlen)
    plan = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
    st = flint_attn_bshd_plan(_ptr(m), _ptr(d), batch, seqlen, _ptr(plan), nbytes,
                              _stream_handle(device))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_bshd_plan")
    info = tuple(int(x) for x in plan[:8].cpu())
    n = info[0]
    cu = plan[8:8 + n + 1]
    seqused = plan[9 + N:9 + N + n]
    pack = plan[9 + 2 * N:9 + 2 * N + info[2]] if info[3] else None
    unpack = plan[9 + 3 * N:9 + 4 * N] if info[3] else None
    return info, cu, seqused, pack, unpack


_NEG_INF_BITS = 0xFF800000  # float32 -inf as a 32-bit word


FLINT_MAX_SEQLEN = 2097152


def _layer_args(q, k, v, q_norm_w, k_norm_w, sinks, positions, cu_seqlens, attention_mask,
                seqused, max_seqlen, dtype=None, document_ids=None, sync=True) -> _Args:
    """Checks the layer's tensors; returns the call's THD description.

    Reads nothing back from the device except, with ``sync`` (the default),
    the counts of the BSHD plan when there is an attention_mask or
    document_ids. Without ``sync``, an attention_mask alone is taken as
    trailing padding (its lengths stay on the device; a row with a hole is
    reported by the forward as a device-data error), and document_ids are
    refused."""
    import torch

    if not q.is_cuda:
        raise ValueError("flint_attn runs on a HIP device; q is on the CPU")
    dev = q.device
    dtype = torch.bfloat16 if dtype is None else dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w), ("sinks", sinks)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev:
            raise TypeError(f"{name} must be a contiguous float32 tensor on {dev}")
    pack = unpack = None
    if q.dim() == 4:
        B, S = q.shape[0], q.shape[1]
        T = B * S
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is for THD input; BSHD takes attention_mask or seqused")
        cu = torch.arange(0, T + 1, max(S, 1), dtype=torch.int32, device=dev)[:B + 1]
        n = B
        mx = S
        if (attention_mask is not None or document_ids is not None) and seqused is not None:
            raise ValueError("pass attention_mask / document_ids or seqused, not both")
        if not sync and document_ids is not None:
            raise ValueError("document_ids need the plan's counts on the host (sync=True)")
        if not sync and attention_mask is not None:
            if tuple(attention_mask.shape) != (B, S):
                raise ValueError("attention_mask must be [batch, seqlen]")
            seqused = seqused_from_mask(attention_mask, check=False)
        elif attention_mask is not None or document_ids is not None:
            info, cu, seqused, pack, unpack = bshd_plan(attention_mask, document_ids, B, S, dev)
            n, mx, T = info[0], info[1], info[2]
            if positions is not None and pack is not None:
                if positions.dtype != torch.int32 or positions.numel() != B * S:
                    raise TypeError("positions must be int32 [batch, seqlen] on the device")
                pp = torch.empty(T, dtype=torch.int32, device=dev)
                _copy_rows(positions.reshape(B * S, 1).contiguous(), pack, T, pp)
                positions = pp
    elif q.dim() == 3:
        T = q.shape[0]
        if attention_mask is not None or document_ids is not None:
            raise ValueError("THD input takes cu_seqlens, not attention_mask or document_ids")
        if cu_seqlens is None:
            cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
            mx = T
        else:
            cu = cu_seqlens
            if cu.dtype != torch.int32 or not cu.is_contiguous() or cu.device != dev:
                raise TypeError("cu_seqlens must be a contiguous int32 tensor on the device")
            # without max_seqlen the bound is T itself (capped at the longest
            # sequence the kernels take); a longer sequence is a device-data error
            mx = max_seqlen if max_seqlen is not None else min(T, FLINT_MAX_SEQLEN)
        n = cu.numel() - 1
    else:
        raise ValueError("q must be [B, S, H, D] or [T, H, D]")
    if seqused is not None and (seqused.dtype != torch.int32 or seqused.device != dev
                                or seqused.numel() != n):
        raise TypeError("seqused must be int32 [n_seqs] on the device")
    if positions is not None:
        if positions.dtype != torch.int32 or positions.device != dev or positions.numel() != T:
            raise TypeError("positions must be int32 with one entry per token, on the device")
        positions = positions.contiguous()
    return _Args(T, n, mx, cu, seqused, positions, pack, unpack)


def flint_attn(q, k, v, q_norm_w, k_norm_w, sinks, *, positions=None, cu_seqlens=None,
               attention_mask=None, document_ids=None, seqused=None,
               max_seqlen: Optional[int] = None, window: int = 513, use_rope: bool = True,
               rope_theta: float = 1.0e6, eps: float = 1.0e-6, out=None, workspace=None,
               return_lse: bool = False, sync: bool = True, check: bool = False):
    """Sink-aware GQA attention forward on torch tensors.

    q: bf16 [B, S, 32, 128] (BSHD) or [T, 32, 128] (THD); k, v: bf16 with 4
    heads in the same layout. q_norm_w, k_norm_w: fp32 [128]; sinks: fp32 [32].
    THD takes ``cu_seqlens`` (int32 [n+1], device) and, optionally,
    ``max_seqlen``; BSHD takes ``attention_mask`` [B, S] (any padding) and/or
    ``document_ids`` [B, S] (documents = runs of equal id among the valid
    tokens), or ``seqused`` [B]. ``positions`` is int32 [B, S] or [T] (default:
    index in the sequence or document). Returns the output in q's layout; with
    ``return_lse`` also the per-row normalizer, float32 [..., 32] in
    natural-log units (what the backward takes; -inf on padding).

    Device-data errors (bad cu_seqlens or seqused, a row of attention_mask with
    a hole under ``sync=False``) are found on the device: the call then writes
    nothing to the output, which holds whatever it held (uninitialized memory
    when the wrapper allocated it). ``check=True`` synchronizes after the call
    and raises FlintError on such an error; otherwise read it with
    ``flint_attn_device_status(workspace)``. ``sync=False`` makes the call read
    nothing back from the device (for HIP graph capture): an attention_mask is
    then taken as trailing padding and document_ids are refused.
    """
    import torch

    a = _layer_args(q, k, v, q_norm_w, k_norm_w, sinks, positions, cu_seqlens, attention_mask,
                    seqused, max_seqlen, document_ids=document_ids, sync=sync)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    qq, kk, vv = a.gather(q), a.gather(k), a.gather(v)
    o = out if a.pack is None else torch.empty_like(qq)
    nbytes = flint_attn_workspace_bytes(a.T, a.n, a.mx, k.shape[-2], k.shape[-1])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(qq), _ptr(kk), _ptr(vv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(sinks),
            _ptr(a.positions), _ptr(a.cu), _ptr(a.seqused), a.n, a.mx, a.T, q.shape[-2],
            k.shape[-2], q.shape[-1], int(window), int(bool(use_rope)), float(rope_theta),
            float(eps), _ptr(workspace), workspace.numel(), _ptr(o))
    if not return_lse:
        st = flint_attn_fwd(*args, _stream_handle(dev))
        if st != FLINT_OK:
            raise FlintError(st, "flint_attn_fwd")
        _check_device(check, workspace, dev)
        return a.scatter(o, out)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ls = lse if a.pack is None else torch.empty((a.T, q.shape[-2]), dtype=torch.float32, device=dev)
    st = flint_attn_fwd_lse(*args, _ptr(ls), _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_fwd_lse")
    _check_device(check, workspace, dev)
    return a.scatter(o, out), a.scatter(ls, lse, fill=_NEG_INF_BITS)


def _check_device(check, workspace, dev):
    """With ``check``: synchronizes and raises on a device-data error of the call."""
    if not check:
        return
    st, flags = flint_attn_device_status(_ptr(workspace), _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, f"flint_attn device data (flags {flags})")


def flint_attn_f16(q, k, v, q_norm_w, k_norm_w, sinks, *, positions=None, cu_seqlens=None,
                   attention_mask=None, document_ids=None, seqused=None,
                   max_seqlen: Optional[int] = None,
                   window: int = 513, use_rope: bool = True, rope_theta: float = 1.0e6,
                   eps: float = 1.0e-6, out=None, workspace=None):
    """The FP16 attention-compute variant on torch tensors: q, k, v float32 (the
    projections) in the layouts of ``flint_attn``; returns float32 output holding
    the fp16-rounded attention result."""
    import torch

    a = _layer_args(q, k, v, q_norm_w, k_norm_w, sinks, positions, cu_seqlens, attention_mask,
                    seqused, max_seqlen, dtype=torch.float32, document_ids=document_ids)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    qq, kk, vv = a.gather(q), a.gather(k), a.gather(v)
    o = out if a.pack is None else torch.empty_like(qq)
    nbytes = flint_attn_f16_workspace_bytes(a.T, a.n, a.mx, k.shape[-2], k.shape[-1])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = flint_attn_fwd_f16(_ptr(qq), _ptr(kk), _ptr(vv), _ptr(q_norm_w), _ptr(k_norm_w),
                            _ptr(sinks), _ptr(a.positions), _ptr(a.cu), _ptr(a.seqused), a.n,
                            a.mx, a.T, q.shape[-2], k.shape[-2], q.shape[-1], int(window),
                            int(bool(use_rope)), float(rope_theta), float(eps), _ptr(workspace),
                            workspace.numel(), _ptr(o), _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_fwd_f16")
    return a.scatter(o, out)


def flint_attn_backward(dout, q, k, v, q_norm_w, k_norm_w, sinks, out, lse, *, positions=None,
                        cu_seqlens=None, attention_mask=None, document_ids=None, seqused=None,
                        max_seqlen: Optional[int] = None, window: int = 513,
                        use_rope: bool = True, rope_theta: float = 1.0e6, eps: float = 1.0e-6,
                        workspace=None):
    """Gradients of the layer for upstream ``dout`` (bf16, the output's layout).

    ``out`` and ``lse`` are what ``flint_attn(..., return_lse=True)`` returned
    for the same inputs. Returns (dq, dk, dv, dq_norm_w, dk_norm_w, dsinks):
    bf16 in the layouts of q, k, v and float32 for the parameters.
    """
    import torch

    a = _layer_args(q, k, v, q_norm_w, k_norm_w, sinks, positions, cu_seqlens, attention_mask,
                    seqused, max_seqlen, document_ids=document_ids)
    dev = q.device
    for name, t, dt in (("dout", dout, torch.bfloat16), ("out", out, torch.bfloat16),
                        ("lse", lse, torch.float32)):
        if t.dtype != dt or not t.is_contiguous() or t.device != dev:
            raise TypeError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if dout.shape != q.shape or out.shape != q.shape or lse.shape != q.shape[:-1]:
        raise ValueError("dout and out must have q's shape and lse q's shape without head_dim")
    qq, kk, vv = a.gather(q), a.gather(k), a.gather(v)
    oo, ll, dd = a.gather(out), a.gather(lse), a.gather(dout)
    dq, dk, dv = torch.empty_like(qq), torch.empty_like(kk), torch.empty_like(vv)
    dqw = torch.empty_like(q_norm_w)
    dkw = torch.empty_like(k_norm_w)
    dsk = torch.empty_like(sinks)
    nbytes = flint_attn_bwd_workspace_bytes(a.T, a.n, a.mx, k.shape[-2], k.shape[-1])
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = flint_attn_bwd(_ptr(qq), _ptr(kk), _ptr(vv), _ptr(q_norm_w), _ptr(k_norm_w),
                        _ptr(sinks), _ptr(a.positions), _ptr(a.cu), _ptr(a.seqused), a.n, a.mx,
                        a.T, q.shape[-2], k.shape[-2], q.shape[-1], int(window),
                        int(bool(use_rope)), float(rope_theta), float(eps), _ptr(oo), _ptr(ll),
                        _ptr(dd), _ptr(workspace), workspace.numel(), _ptr(dq), _ptr(dk),
                        _ptr(dv), _ptr(dqw), _ptr(dkw), _ptr(dsk), _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, "flint_attn_bwd")
    if a.pack is not None:
        dq = a.scatter(dq, torch.empty_like(q))
        dk = a.scatter(dk, torch.empty_like(k))
        dv = a.scatter(dv, torch.empty_like(v))
    return dq, dk, dv, dqw, dkw, dsk


def _check_bf16(name, t, dev, shape=None):
    import torch

    if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != dev:
        raise TypeError(f"{name} must be a contiguous bfloat16 tensor on {dev}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")


def qkv_projection(x, w_q, w_k, w_v):
    """q, k, v = x W^T for hidden states x [..., hidden] (bf16); returns
    q [..., 32, 128], k and v [..., 4, 128] (bf16)."""
    import torch

    dev = x.device
    hidden = x.shape[-1]
    lead = tuple(x.shape[:-1])
    T = int(np.prod(lead)) if lead else 1
    _check_bf16("x", x, dev)
    _check_bf16("w_q", w_q, dev, (NUM_Q_HEADS * HEAD_DIM, hidden))
    _check_bf16("w_k", w_k, dev, (NUM_KV_HEADS * HEAD_DIM, hidden))
    _check_bf16("w_v", w_v, dev, (NUM_KV_HEADS * HEAD_DIM, hidden))
    q = torch.empty(lead + (NUM_Q_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    k = torch.empty(lead + (NUM_KV_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    st = flint_proj_qkv(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), T, hidden, NUM_Q_HEADS,
                        NUM_KV_HEADS, HEAD_DIM, _ptr(q), _ptr(k), _ptr(v), _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, "flint_proj_qkv")
    return q, k, v


def output_projection(o, w_o):
    """y = o W_o^T for the layer's output o [..., 32, 128] (bf16); returns y [..., hidden]."""
    import torch

    dev = o.device
    hidden = w_o.shape[0]
    lead = tuple(o.shape[:-2])
    T = int(np.prod(lead)) if lead else 1
    _check_bf16("o", o, dev)
    _check_bf16("w_o", w_o, dev, (hidden, NUM_Q_HEADS * HEAD_DIM))
    if tuple(o.shape[-2:]) != (NUM_Q_HEADS, HEAD_DIM):
        raise ValueError("o must be [..., 32, 128]")
    y = torch.empty(lead + (hidden,), dtype=torch.bfloat16, device=dev)
    st = flint_proj_out(_ptr(o), _ptr(w_o), T, hidden, NUM_Q_HEADS, HEAD_DIM, _ptr(y),
                        _stream_handle(dev))
    if st != FLINT_OK:
        raise FlintError(st, "flint_proj_out")
    return y


def flint_attention_block(hidden_states, w_q, w_k, w_v, w_o, q_norm_w, k_norm_w, sinks, **layer):
    """FlintAttention.forward: projections, the layer (``flint_attn`` keyword
    arguments: positions, cu_seqlens / attention_mask / document_ids, window,
    use_rope, ...), output projection. hidden_states [B, S, hidden] or
    [T, hidden] bf16; returns the same shape."""
    q, k, v = qkv_projection(hidden_states, w_q, w_k, w_v)
    o = flint_attn(q, k, v, q_norm_w, k_norm_w, sinks, **layer)
    return output_projection(o, w_o)


class KVCache:
    """One layer's KV cache for decode, in the layout the C ABI documents.

    ``k`` [batch, 4, cap/32, 2, 4, 64, 8] and ``vt`` [batch, 4, cap/32, 8, 64, 8]
    bf16 hold the normalized, rotated keys and the values in 32-slot blocks in
    the order the decode kernel reads them (``dense_keys`` / ``dense_values``
    unpack them to [batch, 4, cap, 128]); ``length`` int32 [batch] counts the
    tokens each sequence holds. ``window`` > 0 makes it a ring of the last
    ``window`` tokens (cap is rounded up to a multiple of 32); ``window`` = 0
    keeps ``max_tokens`` tokens.
    """

    def __init__(self, batch: int, window: int, max_tokens: int = 0, *, use_rope: bool = True,
                 rope_theta: float = 1.0e6, eps: float = 1.0e-6, device="cuda"):
        import torch

        need = window if window > 0 else max_tokens
        if need <= 0:
            raise ValueError("a full-attention cache needs max_tokens > 0")
        self.cap = (need + 31) // 32 * 32
        self.batch, self.window = batch, window
        self.use_rope, self.rope_theta, self.eps = use_rope, rope_theta, eps
        nb = self.cap // 32
        self.k = torch.zeros(batch, NUM_KV_HEADS, nb, 2, 4, 64, 8, dtype=torch.bfloat16,
                             device=device)
        self.vt = torch.zeros(batch, NUM_KV_HEADS, nb, 8, 64, 8, dtype=torch.bfloat16,
                              device=device)
        self.length = torch.zeros(batch, dtype=torch.int32, device=device)
        nbytes = flint_attn_decode_workspace_bytes(batch, self.cap)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def dense_keys(self):
        """K' as [batch, 4, cap, 128] (slot-major), unpacked from the blocks."""
        B, nb = self.batch, self.cap // 32
        k = self.k.view(B, NUM_KV_HEADS, nb, 2, 4, 4, 16, 8)  # blk, kh, ds, qd, col, e
        return k.permute(0, 1, 2, 3, 6, 4, 5, 7).reshape(B, NUM_KV_HEADS, self.cap, HEAD_DIM)

    def dense_values(self):
        """V as [batch, 4, cap, 128] (slot-major), unpacked from the blocks."""
        B, nb = self.batch, self.cap // 32
        v = self.vt.view(B, NUM_KV_HEADS, nb, 8, 4, 16, 2, 4)  # blk, db, qd, col, hi, lo
        return v.permute(0, 1, 2, 6, 4, 7, 3, 5).reshape(B, NUM_KV_HEADS, self.cap, HEAD_DIM)

    def _check(self, name, t, dtype, shape):
        import torch

        if t.dtype != dtype or not t.is_contiguous() or t.device != self.k.device:
            raise TypeError(f"{name} must be a contiguous {dtype} tensor on {self.k.device}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")

    def append(self, k, v, k_norm_w, positions=None):
        """Appends k/v [batch, n_new, 4, 128] bf16 (before RMSNorm) to every sequence."""
        import torch

        B, n_new = k.shape[0], k.shape[1]
        self._check("k", k, torch.bfloat16, (self.batch, n_new, NUM_KV_HEADS, HEAD_DIM))
        self._check("v", v, torch.bfloat16, (self.batch, n_new, NUM_KV_HEADS, HEAD_DIM))
        self._check("k_norm_w", k_norm_w, torch.float32, (HEAD_DIM,))
        if positions is not None:
            self._check("positions", positions, torch.int32, (self.batch, n_new))
        st = flint_attn_kv_append(_ptr(k), _ptr(v), _ptr(k_norm_w), _ptr(positions),
                                  _ptr(self.length), B, n_new, _ptr(self.k), _ptr(self.vt),
                                  self.cap, NUM_KV_HEADS, HEAD_DIM, self.window,
                                  int(bool(self.use_rope)), float(self.rope_theta),
                                  float(self.eps), _ptr(self.workspace), self.workspace.numel(),
                                  _stream_handle(k.device))
        if st != FLINT_OK:
            raise FlintError(st, "flint_attn_kv_append")
        self.length += n_new

    def decode(self, q, k, v, q_norm_w, k_norm_w, sinks, positions=None, out=None):
        """One step: q [batch, 32, 128], k/v [batch, 4, 128] bf16 (before RMSNorm).

        Appends the token, returns its attention output [batch, 32, 128] and
        advances the lengths.
        """
        import torch

        self._check("q", q, torch.bfloat16, (self.batch, NUM_Q_HEADS, HEAD_DIM))
        self._check("k", k, torch.bfloat16, (self.batch, NUM_KV_HEADS, HEAD_DIM))
        self._check("v", v, torch.bfloat16, (self.batch, NUM_KV_HEADS, HEAD_DIM))
        for name, t in (("q_norm_w", q_norm_w), ("k_norm_w", k_norm_w)):
            self._check(name, t, torch.float32, (HEAD_DIM,))
        self._check("sinks", sinks, torch.float32, (NUM_Q_HEADS,))
        if positions is not None:
            self._check("positions", positions, torch.int32, (self.batch,))
        if out is None:
            out = torch.empty_like(q)
        st = flint_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w),
                               _ptr(sinks), _ptr(positions), _ptr(self.length), self.batch,
                               _ptr(self.k), _ptr(self.vt), self.cap, NUM_Q_HEADS, NUM_KV_HEADS,
                               HEAD_DIM, self.window, int(bool(self.use_rope)),
                               float(self.rope_theta), float(self.eps), _ptr(self.workspace),
                               self.workspace.numel(), _ptr(out), _stream_handle(q.device))
        if st != FLINT_OK:
            raise FlintError(st, "flint_attn_decode")
        self.length += 1
        return out

    def device_status(self):
        return flint_attn_device_status(_ptr(self.workspace), _stream_handle(self.k.device))
