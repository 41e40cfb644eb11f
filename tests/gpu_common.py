"""Helpers for GPU parity tests: run the HIP path and grade it against the oracle."""

from __future__ import annotations

import numpy as np
import torch

import attention_head_rmsnorm_amd as fa

from .common import f64, i64, oracle_for, seq_index

MAX_ERR_FRAC = 2e-2   # max |O_gpu - O_oracle| <= 2e-2 * max|V|
MEAN_ERR_FRAC = 1e-3  # mean |O_gpu - O_oracle| <= 1e-3 * max|V|


def dev():
    return torch.device("cuda", 0)


def run_gpu(wl, layer, *, sinks=None, positions="keep", bshd=None, workspace=None, out=None):
    """Runs the HIP path on a workload; returns the device output (THD [T, 32, 128])."""
    d = dev()
    q, k, v = wl.q.to(d), wl.k.to(d), wl.v.to(d)
    qw, kw = wl.q_norm_w.to(d), wl.k_norm_w.to(d)
    sk = (wl.sinks if sinks is None else torch.as_tensor(sinks, dtype=torch.float32)).to(d)
    pos = wl.positions if isinstance(positions, str) else positions
    pos = None if pos is None else torch.as_tensor(pos).to(torch.int32).to(d)
    use_bshd = (wl.layout == "bshd") if bshd is None else bshd
    kw_args = dict(window=layer.window, use_rope=layer.use_rope, rope_theta=layer.theta,
                   eps=layer.eps, workspace=workspace)
    if use_bshd:
        B, S = wl.batch, wl.seqlen
        mask = wl.attention_mask()
        o = fa.flint_attn(q.view(B, S, 32, 128), k.view(B, S, 4, 128), v.view(B, S, 4, 128), qw, kw,
                          sk, positions=None if pos is None else pos.view(B, S),
                          attention_mask=None if mask is None else mask.to(d),
                          out=None if out is None else out.view(B, S, 32, 128), **kw_args)
        return o.view(B * S, 32, 128)
    cu = wl.cu_seqlens.to(d)
    su = None if wl.seqused is None else wl.seqused.to(d)
    return fa.flint_attn(q, k, v, qw, kw, sk, positions=pos, cu_seqlens=cu, seqused=su,
                         max_seqlen=wl.max_seqlen, out=out, **kw_args)


def valid_rows(wl):
    T = wl.total_tokens
    s, ell = seq_index(i64(wl.cu_seqlens), T)
    if wl.seqused is None:
        return np.ones(T, bool)
    return ell < i64(wl.seqused)[s]


def grade(got, ref, wl, rows=None, what="", max_frac=MAX_ERR_FRAC, mean_frac=MEAN_ERR_FRAC):
    """Asserts the tolerance on valid rows and exact zeros on padded rows.

    got, ref: [len(rows), 32, 128] (rows=None: every token). Returns stats.
    """
    vmax = float(np.max(np.abs(f64(wl.v)))) if wl.v.numel() else 1.0
    ok = valid_rows(wl)
    if rows is not None:
        ok = ok[np.asarray(rows)]
    g = got.astype(np.float64)
    err = np.abs(g[ok] - ref[ok])
    max_err = float(err.max()) if err.size else 0.0
    mean_err = float(err.mean()) if err.size else 0.0
    stats = dict(max_err=max_err, mean_err=mean_err, vmax=vmax,
                 max_frac=max_err / vmax, mean_frac=mean_err / vmax, rows=int(ok.sum()))
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert max_err <= max_frac * vmax, f"{what}: max err {max_err:.4g} > {max_frac}*{vmax:.4g}"
    assert mean_err <= mean_frac * vmax, f"{what}: mean err {mean_err:.4g} > {mean_frac}*{vmax:.4g}"
    if (~ok).any():
        assert np.all(g[~ok] == 0.0), f"{what}: padded rows are not exact zeros"
    return stats


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_against_oracle(wl, layer, rows=None, **gpu_kw):
    out = run_gpu(wl, layer, **gpu_kw)
    torch.cuda.synchronize()
    got = to_np(out if rows is None else out[torch.as_tensor(rows, device=out.device)])
    sinks = gpu_kw.get("sinks")
    over = {} if sinks is None else {"sinks": np.asarray(sinks, np.float64)}
    pos = gpu_kw.get("positions", "keep")
    if not isinstance(pos, str):
        over["positions"] = None if pos is None else i64(torch.as_tensor(pos))
    ref = oracle_for(wl, layer, rows=rows, **over)
    return grade(got, ref, wl, rows=rows, what=f"{wl.name}/{layer.name}"), out


def with_filler(wl, n_fill=2048, seed=90001):
    """The workload as THD plus one extra seeded document of n_fill tokens.

    THD documents are independent, so the rows of the original sequences keep
    their exact values; the extra document only raises the number of work
    items so that the forward runs on the 8-wave kernel (FLINT_KERNEL_WIDE)
    instead of the split one. BSHD padding becomes THD seqused. Returns
    (workload, rows of the original tokens)."""
    from workload.gen import Workload

    rng = np.random.default_rng(seed)
    T = wl.total_tokens

    def ext(t, shape):
        x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
        return torch.cat([t, x.to(t.dtype)], 0)

    q = ext(wl.q, (n_fill, 32, 128))
    k = ext(wl.k, (n_fill, 4, 128))
    v = ext(wl.v, (n_fill, 4, 128))
    cu = torch.cat([wl.cu_seqlens, torch.tensor([T + n_fill], dtype=torch.int32)])
    su = None
    if wl.seqused is not None:
        su = torch.cat([wl.seqused, torch.tensor([n_fill], dtype=torch.int32)])
    pos = None
    if wl.positions is not None:
        pos = torch.cat([wl.positions, torch.arange(n_fill, dtype=torch.int32)])
    out = Workload(name=wl.name + "+fill", seed=wl.seed, layout="thd", q=q, k=k, v=v,
                   q_norm_w=wl.q_norm_w, k_norm_w=wl.k_norm_w, sinks=wl.sinks, cu_seqlens=cu,
                   seqused=su, positions=pos, layers=list(wl.layers))
    return out, np.arange(T, dtype=np.int64)


def kernel_of(wl):
    """The attention kernel the forward launches for this workload."""
    return fa.flint_attn_fwd_kernel(wl.total_tokens, wl.n_seqs)


def huge_positions(wl, seed=5):
    """The workload with RoPE positions of magnitude 2^24 and more on about
    half of its tokens (both signs, the int32 limits and the values either
    side of 2^24 among them) and small ones on the rest, interleaved, so that
    waves hold both kinds. Positions of magnitude below 2^24 are exact as
    floats, which the fast angle reduction relies on; the others take the
    exact integer reduction lane by lane."""
    rng = np.random.default_rng(seed)
    T = wl.total_tokens
    big = rng.integers(2 ** 24, 2 ** 31, size=T, dtype=np.int64)
    big = np.where(rng.random(T) < 0.5, big, -big)
    small = rng.integers(-(2 ** 20), 2 ** 20, size=T, dtype=np.int64)
    pos = np.where(rng.random(T) < 0.5, big, small)
    edges = [2 ** 24 - 1, 2 ** 24, -(2 ** 24 - 1), -(2 ** 24), 2 ** 31 - 1, -(2 ** 31), 0, -1]
    pos[: min(T, len(edges))] = edges[: min(T, len(edges))]
    wl.positions = torch.from_numpy(np.clip(pos, -(2 ** 31), 2 ** 31 - 1).astype(np.int32))
    return wl
