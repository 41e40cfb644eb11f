"""Benchmark of the Flint sink-attention prefill on one MI355X.

Metric: sink-attention prefill TFLOP/s counting only unmasked FLOPs (QK^T and
PV: 4 * head_dim FLOPs per (query head, allowed key) pair, 32 query heads),
and the attention kernel's fraction of the bf16 dense MFMA peak.

Default workload: full-attention NoPE prefill, batch 1, S = 8192, 32 query /
4 key-value heads, head dim 128, FP32 sinks ~N(0,1), bf16 inputs ~N(0,1) from
a seeded generator, resident in HBM before the timed region. One step = one
flint_attn_fwd call: the preparation launch (schedule and K/V tiles) and the
attention kernel. Before the W warm-up steps the step runs for --settle-ms
(default 300 ms) so that the K timed steps see the GPU's steady clock; the
JSON line records that run ("settle") and a manifest of the run (seed,
SHA-256 of the inputs and of the sources, versions, GPU).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config tstar|c1|c2|c3|c4|c4full|c5]
       python bench.py --decode [--decode-batch B] [--decode-len L] [--decode-window W] [--graph]
                                         (one decode step per sequence over an L-token
                                          KV cache: HBM GB/s against 8 TB/s; --graph
                                          replays the step from a HIP graph)
       python bench.py --backward [--config ...]   (one flint_attn_bwd call per step)
       python bench.py --fp16 [--config ...]       (the FP16 attention-compute variant)
       python bench.py --bshd-docs                 (BSHD rows of packed documents, in place and with holes)
       python bench.py --proj                      (q/k/v and output projections, and the whole block)
       python bench.py --copy-probe     (plain device copy of known size, for
                                          calibrating FETCH_SIZE / WRITE_SIZE)
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sink-attention prefill TFLOP/s (unmasked FLOPs) & % bf16 MFMA peak, 1 GPU"
BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
# the forward attention kernel's sources (its counters go stale when either changes)
KERNEL_SRCS = [os.path.join(ROOT, "attention_head_rmsnorm_amd", "csrc", f)
               for f in ("flint_attn.hip", "flint_common.h")]
TRAFFIC_PROFILES = {
    "tstar": os.path.join(ROOT, "profiles", "attn_kernel_s8192_full_nope_traffic.md"),
    "c3": os.path.join(ROOT, "profiles", "attn_kernel_b8_s8192_sw513_rope_traffic.md"),
    "c1": os.path.join(ROOT, "profiles", "attn_s768_sw513_rope_traffic.md"),
}
COPY_PROBE_BYTES = 1 << 30


def unmasked_pairs(cu, seqused, window):
    """Sum over valid tokens of the number of allowed keys."""
    cu = np.asarray(cu, np.int64)
    total = 0
    for s in range(len(cu) - 1):
        L = int(cu[s + 1] - cu[s])
        u = L if seqused is None else int(seqused[s])
        ell = np.arange(u, dtype=np.int64)
        n = ell + 1 if window == 0 else np.minimum(ell + 1, window)
        total += int(n.sum())
    return total


def pairs_of_rows(cu, seqused, window, rows):
    cu = np.asarray(cu, np.int64)
    rows = np.asarray(rows, np.int64)
    s = np.searchsorted(cu, rows, side="right") - 1
    ell = rows - cu[s]
    u = (cu[s + 1] - cu[s]) if seqused is None else np.asarray(seqused, np.int64)[s]
    n = np.where(ell < u, ell + 1 if window == 0 else np.minimum(ell + 1, window), 0)
    return int(n.sum())


def source_sha256():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(cfg):
    """HBM bytes per attention-kernel launch from the committed PMC summary.

    The summary records the kernel source hash it was taken with; a different
    current source means the counters no longer describe this kernel -> None.
    """
    path = TRAFFIC_PROFILES.get(cfg)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    mh = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    mb = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not mh or not mb or mh.group(1) != source_sha256():
        return None
    return float(mb.group(1))


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(wl, layer, budget_rows):
    """Times the FP64 oracle on an evenly spaced row sample of the workload."""
    from oracle import flint_attention

    T = wl.total_tokens
    step = max(1, T // budget_rows)
    rows = np.arange(step // 2, T, step, dtype=np.int64)[:budget_rows]
    args = dict(q=wl.q.double().numpy(), k=wl.k.double().numpy(), v=wl.v.double().numpy(),
                q_norm_w=wl.q_norm_w.double().numpy(), k_norm_w=wl.k_norm_w.double().numpy(),
                sinks=wl.sinks.double().numpy(), cu_seqlens=wl.cu_seqlens.numpy(),
                seqused=None if wl.seqused is None else wl.seqused.numpy(),
                positions=None if wl.positions is None else wl.positions.numpy(),
                window=layer.window, use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps)
    t0 = time.perf_counter()
    flint_attention(rows=rows, **args)
    dt = time.perf_counter() - t0
    pairs = pairs_of_rows(wl.cu_seqlens.numpy(), None if wl.seqused is None else wl.seqused.numpy(),
                          layer.window, rows)
    flops = 16384.0 * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{len(rows)} evenly spaced query rows of {T} (all 32 heads), "
                      f"{pairs} unmasked token pairs, {dt:.2f} s, FP64 NumPy",
            "seconds": dt}


def copy_probe():
    import torch

    n = COPY_PROBE_BYTES // 2
    x = torch.randn(n, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 3}), flush=True)


class TimingEvent:
    """A HIP event used only to time work on a stream (hipEventDisableSystemFence).

    Recording a default event (torch.cuda.Event) also performs a system-scope
    fence, which writes back and invalidates caches between the launches it
    separates; an event created with hipEventDisableSystemFence skips that
    fence, so timing a kernel inside the timed steps disturbs them less. The
    elapsed time is read only after a full synchronization of the device.
    Same record / elapsed_time interface as torch.cuda.Event.
    """

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes

        if TimingEvent._hip is None:
            # the HIP runtime torch has loaded (same soname as the library's)
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._ev = ctypes.c_void_p()
        self._check(TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._ev), self.FLAGS),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def record(self, stream):
        self._check(TimingEvent._hip.hipEventRecord(self._ev, stream.cuda_stream), "hipEventRecord")

    def elapsed_time(self, end):
        import ctypes

        ms = ctypes.c_float()
        self._check(TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev),
                    "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        if self._ev and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(self._ev)


def settle(fn, args):
    """Runs fn until args.settle_ms of wall time have passed (synchronizing
    every 10 calls), before the warm-up steps.

    The GPU raises its clock over the first ~100 ms of sustained load: on one
    box the default workload measured 1006 TFLOP/s with 20 steps after 5
    warm-up steps from idle, 1100 after 50 warm-up steps... and 1146 after
    200 steps and 50 warm-ups. Settling first makes the K timed steps measure
    the steady throughput whatever K and W are; the timed region is unchanged
    (exactly K whole steps). Returns what was run, for the JSON line."""
    import torch

    ms = max(0.0, float(args.settle_ms))
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms and n < 100000:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n}


def tensor_sha256(*tensors):
    """SHA-256 over the bytes of the given host or device tensors, in order."""
    import torch

    h = hashlib.sha256()
    for t in tensors:
        if t is None:
            h.update(b"none")
            continue
        c = t.detach().contiguous().cpu()
        h.update(str(tuple(c.shape)).encode() + str(c.dtype).encode())
        h.update(c.view(torch.uint8).numpy().tobytes() if c.numel() else b"")
    return h.hexdigest()


def sources_sha256():
    """SHA-256 over every source the measured library and this script are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_head_rmsnorm_amd", "csrc")
    paths = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    paths += [os.path.join(ROOT, "include", "flint_attn.h"), os.path.abspath(__file__)]
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + f.read())
    return h.hexdigest()


def manifest(seed=None, inputs=None):
    """What the run was: the seeds, hashes of the inputs and of the sources,
    the software versions and the GPU (the record a numerical comparison keeps)."""
    import platform
    import subprocess

    import torch

    git = None
    try:
        git = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except Exception:
        pass
    props = torch.cuda.get_device_properties(0)
    rec = {
        "seed": seed,
        "inputs_sha256": inputs,
        "sources_sha256": sources_sha256(),
        "git_head": git,
        "torch": torch.__version__,
        "hip": getattr(torch.version, "hip", None),
        "python": platform.python_version(),
        "gpu": torch.cuda.get_device_name(0),
        "gpu_arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "gpu_max_clock_mhz": getattr(props, "clock_rate", 0) / 1000.0 or None,
        "host_cpus": os.cpu_count(),
    }
    return rec


def decode_bench(args):
    """Decode step: append the new token, attend over the cache, merge the splits.

    The cache holds decode_len tokens per sequence (filled with kv_append from
    seeded N(0,1) keys and values); every timed step decodes token decode_len
    of every sequence (the same slot each time, so the length stays fixed).
    Algorithmic HBM bytes per step: the cached K' and V^T the step reads, 2 KiB
    per attended token per sequence (4 kv heads x 128 channels x 2 bytes x 2),
    plus q, k, v and out of the new token.
    """
    import torch

    import attention_head_rmsnorm_amd as fa
    from workload.gen import _bf16, _draw_params

    B, L, W = args.decode_batch, args.decode_len, args.decode_window
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(2001)
    qw, kw, sinks = _draw_params(rng, 1.0)
    use_rope = W > 0
    cache = fa.KVCache(B, W, max_tokens=L + 1, use_rope=use_rope, device=dev)
    qw, kw, sinks = qw.to(dev), kw.to(dev), sinks.to(dev)
    chunk = cache.cap if W > 0 else L
    for c0 in range(0, L, chunk):
        n = min(chunk, L - c0)
        k = _bf16(rng.standard_normal((B, n, 4, 128), dtype=np.float32)).to(dev)
        v = _bf16(rng.standard_normal((B, n, 4, 128), dtype=np.float32)).to(dev)
        cache.append(k, v, kw)
    q = _bf16(rng.standard_normal((B, 32, 128), dtype=np.float32)).to(dev)
    k1 = _bf16(rng.standard_normal((B, 4, 128), dtype=np.float32)).to(dev)
    v1 = _bf16(rng.standard_normal((B, 4, 128), dtype=np.float32)).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    p = lambda t: int(t.data_ptr())  # noqa: E731
    call = [p(q), p(k1), p(v1), p(qw), p(kw), p(sinks), 0, p(cache.length), B, p(cache.k),
            p(cache.vt), cache.cap, 32, 4, 128, W, int(use_rope), 1.0e6, 1.0e-6,
            p(cache.workspace), cache.workspace.numel(), p(out), int(stream.cuda_stream)]
    settled = settle(lambda: fa.flint_attn_decode(*call), args)
    for _ in range(args.warmup):
        fa.flint_attn_decode(*call)
    torch.cuda.synchronize()
    st, flags = cache.device_status()
    if st != 0:
        raise RuntimeError(f"decode device error flags {flags}")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    graph = None
    if args.graph:
        # the whole step (its four launches) captured once and replayed: what a
        # serving loop pays once launch overhead is gone
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st = fa.flint_attn_decode(*call[:-1], int(torch.cuda.current_stream(dev).cuda_stream))
        if st != 0:
            raise RuntimeError(fa.flint_attn_strerror(st))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
            continue
        st = fa.flint_attn_decode(*call)
        if st != 0:
            raise RuntimeError(fa.flint_attn_strerror(st))
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    attended = min(L + 1, W) if W > 0 else L + 1
    alg = B * (attended * 2048.0 + (32 + 4 + 4 + 32) * 256.0)
    gbs = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "decode step HBM GB/s (one token per sequence, KV cache read once)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 cache contents, q, k, v)",
        "config": {"workload": f"decode, batch {B}, {L} cached tokens, "
                               + (f"sliding window {W} (RoPE)" if W else "full attention (NoPE)")
                               + (", replayed from a HIP graph" if args.graph else ""),
                   "batch": B, "cached_tokens": L, "window": W, "attended_tokens": attended,
                   "cache_cap": cache.cap, "hip_graph": bool(args.graph)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": alg, "traffic": None},
    }
    if not args.no_cpu_baseline:
        # the oracle's decode: the last row of a sequence of attended tokens
        from oracle import flint_attention

        n_seq = B  # every sequence of the batch
        rng = np.random.default_rng(2002)
        qkv = [rng.standard_normal((attended, h, 128)) for h in (32, 4, 4)]
        t0c = time.perf_counter()
        for _ in range(n_seq):
            flint_attention(qkv[0], qkv[1], qkv[2], f64np(qw), f64np(kw), f64np(sinks),
                            np.array([0, attended]), window=W, use_rope=use_rope,
                            rows=np.array([attended - 1]))
        dt = time.perf_counter() - t0c
        rec["cpu_baseline"] = {"value": round(n_seq * (attended * 2048.0 + 72 * 256.0) / dt / 1e9, 6),
                               "unit": "GB/s", "cores": cpu_threads(), "kind": "oracle",
                               "sample": f"{n_seq} sequences of {attended} attended tokens, the last "
                                         f"row each, {dt:.2f} s, FP64 NumPy"}
    print(json.dumps(rec), flush=True)


def f64np(t):
    return t.detach().double().cpu().numpy()


def backward_bench(args):
    """Backward of one layer: dq, dk, dv, the norm-weight and sink gradients.

    The forward (with its row normalizer) runs once, untimed; every timed step
    is one flint_attn_bwd call over the whole workload. Algorithmic FLOPs are
    the usual 2.5x the forward's (five 2*128-FLOP products per unmasked
    (query, key, head) pair: the logit recompute, dP, dV, dK and dQ); the
    kernels execute 3.5x (the query-major dQ pass recomputes the logits and dP).
    """
    import torch

    import attention_head_rmsnorm_amd as fa
    from workload import make_workload
    from workload.gen import draw_dout

    cfg = args.config
    li = 0
    if cfg == "c4full":
        cfg, li = "c4", 1
    wl = make_workload(cfg)
    layer = wl.layers[li]
    dev = torch.device("cuda", 0)
    fa.load_library()
    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    qw, kw, sk = wl.q_norm_w.to(dev), wl.k_norm_w.to(dev), wl.sinks.to(dev)
    cu = wl.cu_seqlens.to(dev)
    su = None if wl.seqused is None else wl.seqused.to(dev)
    pos = None if wl.positions is None else wl.positions.to(dev)
    T, n, mx = wl.total_tokens, wl.n_seqs, wl.max_seqlen
    kw_args = dict(positions=pos, cu_seqlens=cu, seqused=su, max_seqlen=mx, window=layer.window,
                   use_rope=layer.use_rope, rope_theta=layer.theta, eps=layer.eps)
    out, lse = fa.flint_attn(q, k, v, qw, kw, sk, return_lse=True, **kw_args)
    dout = draw_dout(wl.seed, T).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dqw, dkw, dsk = torch.empty_like(qw), torch.empty_like(kw), torch.empty_like(sk)
    nbytes = fa.flint_attn_bwd_workspace_bytes(T, n, mx)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    call = [p(q), p(k), p(v), p(qw), p(kw), p(sk), p(pos), p(cu), p(su), n, mx, T, 32, 4, 128,
            layer.window, int(layer.use_rope), layer.theta, layer.eps, p(out), p(lse), p(dout),
            p(ws), nbytes, p(dq), p(dk), p(dv), p(dqw), p(dkw), p(dsk), int(stream.cuda_stream)]
    settled = settle(lambda: fa.flint_attn_bwd(*call), args)
    for _ in range(args.warmup):
        st = fa.flint_attn_bwd(*call)
        if st != 0:
            raise RuntimeError(fa.flint_attn_strerror(st))
    torch.cuda.synchronize()
    st, flags = fa.flint_attn_device_status(p(ws), int(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"device data error flags {flags}")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        fa.flint_attn_bwd(*call)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps
    pairs = unmasked_pairs(wl.cu_seqlens.numpy(), None if wl.seqused is None else wl.seqused.numpy(),
                           layer.window)
    flops = 2.5 * 16384.0 * pairs
    value = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "sink-attention backward TFLOP/s (2.5x the forward's unmasked FLOPs), 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v and dO, N(1,0.1) norm weights, N(0,1) sinks)",
        "config": {"workload": wl.description, "name": wl.name, "layer": layer.name,
                   "total_tokens": T, "n_seqs": n, "window": layer.window,
                   "use_rope": layer.use_rope},
        "pct_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "algorithmic_flops": flops,
        "executed_mfma_tflops": round(3.5 * 16384.0 * pairs / (ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "flint_attn_bwd (all its kernels, one call)",
                     "achieved": round(value, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / BF16_PEAK_TFLOPS, 4), "traffic": None},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        # the backward oracle on the workload's first 2,048 tokens as one sequence
        from oracle import flint_attention_backward

        n = min(2048, T)
        sl = slice(0, n)
        t0c = time.perf_counter()
        flint_attention_backward(f64np(wl.q[sl]), f64np(wl.k[sl]), f64np(wl.v[sl]),
                                 f64np(wl.q_norm_w), f64np(wl.k_norm_w), f64np(wl.sinks),
                                 np.array([0, n]), f64np(dout[sl]), window=layer.window,
                                 use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps)
        dt = time.perf_counter() - t0c
        pc = unmasked_pairs(np.array([0, n]), None, layer.window)
        rec["cpu_baseline"] = {"value": round(2.5 * 16384.0 * pc / dt / 1e12, 6),
                               "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
                               "sample": f"the first {n} tokens as one sequence, every gradient, "
                                         f"{pc} unmasked pairs, {dt:.2f} s, FP64 NumPy"}
    print(json.dumps(rec), flush=True)


def fp16_bench(args):
    """The FP16 attention-compute variant: FP32 projections in, fp16 products,
    FP32 output. One step = one flint_attn_fwd_f16 call (schedule, K/V and
    query preparation, attention kernel); FLOPs counted as for the bf16 path."""
    import torch

    import attention_head_rmsnorm_amd as fa
    from workload import make_workload

    cfg = args.config
    li = 0
    if cfg == "c4full":
        cfg, li = "c4", 1
    wl = make_workload(cfg)
    layer = wl.layers[li]
    dev = torch.device("cuda", 0)
    fa.load_library()
    q, k, v = wl.q.float().to(dev), wl.k.float().to(dev), wl.v.float().to(dev)
    qw, kw, sk = wl.q_norm_w.to(dev), wl.k_norm_w.to(dev), wl.sinks.to(dev)
    cu = wl.cu_seqlens.to(dev)
    su = None if wl.seqused is None else wl.seqused.to(dev)
    pos = None if wl.positions is None else wl.positions.to(dev)
    T, n, mx = wl.total_tokens, wl.n_seqs, wl.max_seqlen
    out = torch.empty_like(q)
    nbytes = fa.flint_attn_f16_workspace_bytes(T, n, mx)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    call = [p(q), p(k), p(v), p(qw), p(kw), p(sk), p(pos), p(cu), p(su), n, mx, T, 32, 4, 128,
            layer.window, int(layer.use_rope), layer.theta, layer.eps, p(ws), nbytes, p(out),
            int(stream.cuda_stream)]
    settled = settle(lambda: fa.flint_attn_fwd_f16(*call), args)
    for _ in range(args.warmup):
        st = fa.flint_attn_fwd_f16(*call)
        if st != 0:
            raise RuntimeError(fa.flint_attn_strerror(st))
    torch.cuda.synchronize()
    st, flags = fa.flint_attn_device_status(p(ws), int(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"device data error flags {flags}")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        fa.flint_attn_fwd_f16(*call)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps
    pairs = unmasked_pairs(wl.cu_seqlens.numpy(), None if wl.seqused is None else wl.seqused.numpy(),
                           layer.window)
    flops = 16384.0 * pairs
    value = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "sink-attention prefill TFLOP/s (unmasked FLOPs), FP16 attention compute, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) FP32 q/k/v, N(1,0.1) norm weights, N(0,1) sinks)",
        "config": {"workload": wl.description, "name": wl.name, "layer": layer.name,
                   "total_tokens": T, "n_seqs": n, "window": layer.window,
                   "use_rope": layer.use_rope},
        "pct_f16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "unmasked_flops": flops,
        "roofline": {"bound": "mfma", "kernel": "flint_attn_fwd_f16 (one call)",
                     "achieved": round(value, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / BF16_PEAK_TFLOPS, 4), "traffic": None},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, layer, min(args.cpu_rows, 2048))
        rec["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2)
                               for k2, v2 in cb.items() if k2 != "seconds"}
    print(json.dumps(rec), flush=True)


def bshd_docs_bench(args):
    """BSHD rows of packed documents on a sliding layer (513, RoPE): B=8 rows of
    S=8192 tokens, document lengths log-uniform in [64, 8192] (a packed
    long-context batch), and the same rows with 2% of the tokens masked out
    inside documents. One step = the plan kernel, then the attention call
    (in place), or plan + gather of q, k, v + attention + scatter of the output
    (holes). The plan's counts are read once before timing, as a training loop
    reads them once per batch."""
    import torch

    import attention_head_rmsnorm_amd as fa
    from workload import make_custom
    from workload.gen import SLIDING

    B, S = 8, 8192
    rng = np.random.default_rng(2024)
    ids = np.zeros((B, S), np.int32)
    for b in range(B):
        lens, left = [], S
        while left > 0:
            n = int(min(left, np.exp(rng.uniform(np.log(64), np.log(S)))))
            lens.append(n)
            left -= n
        ids[b] = np.repeat(np.arange(len(lens)), lens)
    holes = np.ones((B, S), np.uint8)
    holes[rng.random((B, S)) < 0.02] = 0
    wl = make_custom(2024, [S] * B, layout="bshd")
    layer = SLIDING
    dev = torch.device("cuda", 0)
    fa.load_library()
    q = wl.q.to(dev).view(B, S, 32, 128)
    k = wl.k.to(dev).view(B, S, 4, 128)
    v = wl.v.to(dev).view(B, S, 4, 128)
    qw, kw, sk = wl.q_norm_w.to(dev), wl.k_norm_w.to(dev), wl.sinks.to(dev)
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    ids_t = torch.from_numpy(ids).to(dev)
    recs = {}
    for name, mask in (("in_place", None), ("holes_2pct", holes)):
        m_t = None if mask is None else torch.from_numpy(mask).to(dev)
        info, cu, su, pack, unpack = fa.bshd_plan(m_t, ids_t, B, S, dev)
        n, mx, T, packed = info[:4]
        nbytes = fa.flint_attn_bshd_plan_bytes(B, S)
        plan = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
        wsb = fa.flint_attn_workspace_bytes(T, n, mx)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        # the plan the timed steps rewrite holds the same description as `cu`, `su`
        pcu = plan[8:8 + n + 1]
        psu = plan[9 + B * S:9 + B * S + n]
        ppk = plan[9 + 2 * B * S:]
        pup = plan[9 + 3 * B * S:]
        qq = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev) if packed else q
        kk = torch.empty((T, 4, 128), dtype=torch.bfloat16, device=dev) if packed else k
        vv = torch.empty((T, 4, 128), dtype=torch.bfloat16, device=dev) if packed else v
        oo = torch.empty((T, 32, 128), dtype=torch.bfloat16, device=dev) if packed else None
        out = torch.empty_like(q)

        def step():
            st = fa.flint_attn_bshd_plan(p(m_t), p(ids_t), B, S, p(plan), nbytes, sh)
            if packed:
                st |= fa.flint_attn_copy_rows(p(q), p(ppk), T, 8192, 0, p(qq), sh)
                st |= fa.flint_attn_copy_rows(p(k), p(ppk), T, 1024, 0, p(kk), sh)
                st |= fa.flint_attn_copy_rows(p(v), p(ppk), T, 1024, 0, p(vv), sh)
            st |= fa.flint_attn_fwd(p(qq), p(kk), p(vv), p(qw), p(kw), p(sk), 0, p(pcu), p(psu), n,
                                    mx, T, 32, 4, 128, layer.window, 1, layer.theta, layer.eps,
                                    p(ws), wsb, p(oo if packed else out), sh)
            if packed:
                st |= fa.flint_attn_copy_rows(p(oo), p(pup), B * S, 8192, 0, p(out), sh)
            if st != 0:
                raise RuntimeError("BSHD documents step failed")

        settled = settle(step, args)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(args.steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        pairs = unmasked_pairs(cu.cpu().numpy(), su.cpu().numpy(), layer.window)
        recs[name] = {"ms_per_step": round(ms, 5), "tflops": round(16384.0 * pairs / (ms * 1e-3) / 1e12, 3),
                      "n_seqs": n, "total_tokens": T, "packed": bool(packed),
                      "valid_tokens": info[4], "documents": info[5]}
    rec = {
        "metric": "sink-attention prefill TFLOP/s (unmasked FLOPs), BSHD packed documents, 1 GPU",
        "value": recs["in_place"]["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": recs["in_place"]["ms_per_step"],
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v; document lengths log-uniform 64..8192)",
        "config": {"workload": "BSHD B=8 S=8192 packed documents, sliding 513 RoPE",
                   "window": layer.window, "use_rope": True},
        "variants": recs,
        "roofline": {"bound": "mfma", "kernel": "plan + flint_attn_fwd, in place (one step)",
                     "achieved": recs["in_place"]["tflops"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": round(recs["in_place"]["tflops"] / BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        # the THD oracle on sampled rows of the documents (in place, no holes)
        from oracle import flint_attention

        info, cu, su, _, _ = fa.bshd_plan(None, ids_t, B, S, dev)
        cu_np = cu.cpu().numpy().astype(np.int64)
        rows = np.arange(0, B * S, 64, dtype=np.int64)
        t0c = time.perf_counter()
        flint_attention(f64np(wl.q), f64np(wl.k), f64np(wl.v), f64np(wl.q_norm_w),
                        f64np(wl.k_norm_w), f64np(wl.sinks), cu_np, window=layer.window,
                        use_rope=True, theta=layer.theta, eps=layer.eps, rows=rows)
        dt = time.perf_counter() - t0c
        pc = pairs_of_rows(cu_np, None, layer.window, rows)
        rec["cpu_baseline"] = {"value": round(16384.0 * pc / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": cpu_threads(), "kind": "oracle",
                               "sample": f"every 64th of {B * S} query rows over the "
                                         f"{info[5]} documents, {pc} unmasked pairs, {dt:.2f} s, "
                                         "FP64 NumPy"}
    print(json.dumps(rec), flush=True)


def proj_bench(args):
    """The projections at 8,192 tokens (hidden 2048): the q/k/v GEMM
    (2048 -> 4096 + 512 + 512) and the output GEMM (4096 -> 2048), each timed
    with HIP events on the launch stream; torch's bf16 linear (hipBLASLt) on the
    same operands timed beside them for context; and the whole attention block
    (projections + the full-attention NoPE layer) per step."""
    import torch

    import attention_head_rmsnorm_amd as fa
    from workload import draw_block, make_workload

    wl = make_workload("tstar")
    layer = wl.layers[0]
    T = wl.total_tokens
    dev = torch.device("cuda", 0)
    fa.load_library()
    x, w_q, w_k, w_v, w_o = (t.to(dev) for t in draw_block(wl.seed, T))
    q = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(T, 4, 128, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    y = torch.empty(T, 2048, dtype=torch.bfloat16, device=dev)
    qw, kw, sk = wl.q_norm_w.to(dev), wl.k_norm_w.to(dev), wl.sinks.to(dev)
    cu = wl.cu_seqlens.to(dev)
    nbytes = fa.flint_attn_workspace_bytes(T, 1, T)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731

    def qkv():
        if fa.flint_proj_qkv(p(x), p(w_q), p(w_k), p(w_v), T, 2048, 32, 4, 128, p(q), p(k), p(v), sh):
            raise RuntimeError("flint_proj_qkv failed")

    def out_proj():
        if fa.flint_proj_out(p(o), p(w_o), T, 2048, 32, 128, p(y), sh):
            raise RuntimeError("flint_proj_out failed")

    def attn():
        if fa.flint_attn_fwd(p(q), p(k), p(v), p(qw), p(kw), p(sk), 0, p(cu), 0, 1, T, T, 32, 4, 128,
                             layer.window, int(layer.use_rope), layer.theta, layer.eps, p(ws), nbytes,
                             p(o), sh):
            raise RuntimeError("flint_attn_fwd failed")

    w_qkv = torch.cat([w_q, w_k, w_v], 0)

    def torch_qkv():
        torch.nn.functional.linear(x, w_qkv)

    def torch_out():
        torch.nn.functional.linear(o.view(T, -1), w_o)

    def timed(fn, steps):
        for _ in range(max(args.warmup, 20)):  # the clocks settle under a steady GEMM load
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    f_qkv = 2.0 * T * 2048 * 5120
    f_out = 2.0 * T * 4096 * 2048
    ms = {name: timed(fn, args.steps) for name, fn in
          (("qkv", qkv), ("out", out_proj), ("torch_qkv", torch_qkv), ("torch_out", torch_out))}
    ms["block"] = timed(lambda: (qkv(), attn(), out_proj()), args.steps)
    attn_flops = 16384.0 * unmasked_pairs(wl.cu_seqlens.numpy(), None, layer.window)
    tf = lambda f, t: f / (t * 1e-3) / 1e12  # noqa: E731
    rec = {
        "metric": "attention-block projections TFLOP/s (q/k/v and output GEMMs), 1 GPU",
        "value": round(tf(f_qkv + f_out, ms["qkv"] + ms["out"]), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms["qkv"] + ms["out"], 5),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 hidden states, N(0,0.02) bf16 weights)",
        "config": {"workload": "8192 tokens, hidden 2048 -> q 4096 + k 512 + v 512, o 4096 -> 2048",
                   "tokens": T},
        "qkv_ms": round(ms["qkv"], 5), "qkv_tflops": round(tf(f_qkv, ms["qkv"]), 3),
        "out_ms": round(ms["out"], 5), "out_tflops": round(tf(f_out, ms["out"]), 3),
        "torch_linear_qkv_ms": round(ms["torch_qkv"], 5),
        "torch_linear_out_ms": round(ms["torch_out"], 5),
        "block_ms": round(ms["block"], 5),
        "block_tflops": round(tf(f_qkv + f_out + attn_flops, ms["block"]), 3),
        "roofline": {"bound": "mfma", "kernel": "proj_gemm_kernel (q/k/v)",
                     "achieved": round(tf(f_qkv, ms["qkv"]), 3), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf(f_qkv, ms["qkv"]) / BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        # the oracle's projections (FP64 products) on every token
        from oracle import linear

        xs = f64np(x)
        wq, wk, wv, wo = (f64np(w) for w in (w_q, w_k, w_v, w_o))
        t0c = time.perf_counter()
        yq = linear(xs, wq)
        linear(xs, wk)
        linear(xs, wv)
        linear(yq, wo)
        dt = time.perf_counter() - t0c
        n = xs.shape[0]
        rec["cpu_baseline"] = {"value": round(n * 2.0 * (2048 * 5120 + 4096 * 2048) / dt / 1e12, 6),
                               "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
                               "sample": f"all {n} tokens, both projections, "
                                         f"{dt:.2f} s, FP64 NumPy"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="tstar")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step this long before the warm-up steps (GPU clock ramp); 0 = off")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--torch-events", action="store_true",
                    help="time each attention launch with torch's default events (system fence) "
                         "instead of fence-free HIP events")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--fp16", action="store_true")
    ap.add_argument("--bshd-docs", action="store_true")
    ap.add_argument("--proj", action="store_true")
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--decode-len", type=int, default=8192)
    ap.add_argument("--decode-window", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: capture one step in a HIP graph and time its replays")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this implementation runs on one GPU only (no cross-GPU sharding); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe()
        return
    if args.decode:
        decode_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.fp16:
        fp16_bench(args)
        return
    if args.bshd_docs:
        bshd_docs_bench(args)
        return
    if args.proj:
        proj_bench(args)
        return

    import attention_head_rmsnorm_amd as fa
    from workload import make_workload

    cfg = args.config
    li = 0
    if cfg == "c4full":
        cfg, li = "c4", 1
    wl = make_workload(cfg)
    layer = wl.layers[li]
    dev = torch.device("cuda", 0)
    fa.load_library()

    q, k, v = wl.q.to(dev), wl.k.to(dev), wl.v.to(dev)
    qw, kw, sk = wl.q_norm_w.to(dev), wl.k_norm_w.to(dev), wl.sinks.to(dev)
    cu = wl.cu_seqlens.to(dev)
    su = None if wl.seqused is None else wl.seqused.to(dev)
    pos = None if wl.positions is None else wl.positions.to(dev)
    T, n, mx = wl.total_tokens, wl.n_seqs, wl.max_seqlen
    out = torch.empty_like(q)
    nbytes = fa.flint_attn_workspace_bytes(T, n, mx)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    p = lambda t: 0 if t is None else int(t.data_ptr())  # noqa: E731
    call_args = [p(q), p(k), p(v), p(qw), p(kw), p(sk), p(pos), p(cu), p(su), n, mx, T, 32, 4, 128,
                 layer.window, int(layer.use_rope), layer.theta, layer.eps, p(ws), nbytes, p(out), sh]

    def step(ev=None):
        if ev is None:
            st = fa.flint_attn_fwd_phases(*call_args, fa.FLINT_PHASE_ALL)
        else:
            st = fa.flint_attn_fwd_phases(*call_args, fa.FLINT_PHASE_SCHEDULE | fa.FLINT_PHASE_KV)
            ev[0].record(stream)
            st |= fa.flint_attn_fwd_phases(*call_args, fa.FLINT_PHASE_ATTEND)
            ev[1].record(stream)
        if st != 0:
            raise RuntimeError(f"flint_attn_fwd_phases failed: {fa.flint_attn_strerror(st)}")

    settled = settle(step, args)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st, flags = fa.flint_attn_device_status(p(ws), sh)
    if st != 0:
        raise RuntimeError(f"device data error flags {flags}")

    K = args.steps
    evs = None
    if not args.torch_events:
        try:
            evs = [(TimingEvent(), TimingEvent()) for _ in range(K)]
        except (OSError, RuntimeError) as e:  # no fence-free events here: torch's instead
            print(f"fence-free HIP events unavailable ({e}); timing with torch.cuda.Event", file=sys.stderr)
            args.torch_events = True
    if evs is None:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / K
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    pairs = unmasked_pairs(wl.cu_seqlens.numpy(), None if wl.seqused is None else wl.seqused.numpy(),
                           layer.window)
    flops = 16384.0 * pairs
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    alg_bytes = 18432.0 * T
    traffic = traffic_from_profile(wl.name if li == 0 else None)
    # bf16 ridge: 2516.6 TFLOP/s / 8 TB/s = 315 FLOP per byte
    intensity = flops / alg_bytes
    bound = "mfma" if intensity >= BF16_PEAK_TFLOPS / (HBM_PEAK_GBS / 1000.0) else "hbm"
    alg_gbs = alg_bytes / (attn_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, N(1,0.1) norm weights, N(0,1) FP32 sinks)",
        "config": {
            "workload": wl.description,
            "name": wl.name,
            "layer": layer.name,
            "batch": wl.batch if wl.layout == "bshd" else None,
            "seq_len": wl.seqlen if wl.layout == "bshd" else None,
            "total_tokens": T,
            "n_seqs": n,
            "window": layer.window,
            "use_rope": layer.use_rope,
            "q_heads": 32,
            "kv_heads": 4,
            "head_dim": 128,
            "parallelism": "single GPU",
        },
        "pct_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "unmasked_flops": flops,
        "attn_kernel_ms": round(attn_ms, 5),
        "prologue_ms": round(ms_step - attn_ms, 5),
        "roofline": {
            "bound": bound,
            "achieved": round(attn_tflops if bound == "mfma" else alg_gbs, 3),
            "peak": BF16_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round(attn_tflops / BF16_PEAK_TFLOPS if bound == "mfma" else alg_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": ("attn_half_kernel" if fa.flint_attn_fwd_kernel(T, n) == fa.FLINT_KERNEL_SPLIT
                       else "attn_kernel"),
            "algorithmic_bytes": alg_bytes,
            "algorithmic_flops": flops,
            "intensity_flop_per_byte": round(intensity, 1),
            "attn_tflops": round(attn_tflops, 3),
            "algorithmic_GBs": round(alg_gbs, 1),
            "traffic_GBs": None if traffic is None else round(traffic / (attn_ms * 1e-3) / 1e9, 1),
        },
        "wall_s_timed": round(wall, 4),
        "kernel_timing": ("torch.cuda.Event per attention launch" if args.torch_events else
                          "hipEventDisableSystemFence events per attention launch"),
        "settle": settled,
        "manifest": manifest(seed=wl.seed, inputs=tensor_sha256(wl.q, wl.k, wl.v, wl.q_norm_w, wl.k_norm_w,
                                                                 wl.sinks, wl.cu_seqlens, wl.seqused,
                                                                 wl.positions)),
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, layer, args.cpu_rows)
        rec["cpu_baseline"] = {k2: (round(v2, 6) if isinstance(v2, float) else v2)
                               for k2, v2 in cb.items() if k2 != "seconds"}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
