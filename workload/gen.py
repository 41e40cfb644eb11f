"""Seeded generators for the layer's synthetic workloads.

Shapes follow the Flint attention layout stated on the NeMo AutoModel "flint"
page (section "Model Architecture"): 32 query heads, 4 key/value heads, head
dimension 128; the sliding window holds 513 keys (the current token and 512
before it); sliding layers use NeoX RoPE, full layers use none. Layouts are the
BSHD / THD forms documented for ``FlintAttention._apply_rope`` and
``FlintAttention.forward`` on the ``flint.layers`` API page.

Every tensor is drawn from one ``numpy.random.default_rng(seed)`` per workload
in a fixed order:

1. structure: per-sequence trailing padding (BSHD) or document lengths (THD);
2. q, k, v as float32 standard normals, rounded to bfloat16 (round to nearest
   even, done by ``torch.Tensor.to``);
3. q_norm_w, k_norm_w ~ N(1, 0.1) and sinks ~ N(0, sink_std) in float32;
4. value modifiers: massive-activation tokens in v (scaled before the bfloat16
   rounding) and pinned sink heads.

Nothing here computes any part of the attention layer.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

NUM_Q_HEADS = 32
NUM_KV_HEADS = 4
HEAD_DIM = 128
SLIDING_WINDOW = 513
ROPE_THETA = 1.0e6
RMS_EPS = 1.0e-6


@dataclass(frozen=True)
class Layer:
    """The per-layer flags of the attention call."""

    window: int  # keys per query including the current token; 0 = full causal
    use_rope: bool
    theta: float = ROPE_THETA
    eps: float = RMS_EPS

    @property
    def name(self) -> str:
        return f"sw{self.window}-rope" if self.window else "full-nope"


SLIDING = Layer(window=SLIDING_WINDOW, use_rope=True)
FULL = Layer(window=0, use_rope=False)


@dataclass
class Workload:
    name: str
    seed: int
    layout: str  # "bshd" or "thd"
    q: torch.Tensor  # bf16 [T, 32, 128] (BSHD flattened to T = B*S)
    k: torch.Tensor  # bf16 [T, 4, 128]
    v: torch.Tensor  # bf16 [T, 4, 128]
    q_norm_w: torch.Tensor  # f32 [128]
    k_norm_w: torch.Tensor  # f32 [128]
    sinks: torch.Tensor  # f32 [32]
    cu_seqlens: torch.Tensor  # int32 [n+1]
    seqused: Optional[torch.Tensor]  # int32 [n] valid prefix length, or None
    positions: Optional[torch.Tensor]  # int32 [T], or None (= index in sequence)
    layers: List[Layer]
    batch: int = 0  # BSHD only
    seqlen: int = 0  # BSHD only
    description: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.numel() - 1)

    @property
    def max_seqlen(self) -> int:
        cu = self.cu_seqlens.to(torch.int64)
        if cu.numel() < 2:
            return 0
        return int((cu[1:] - cu[:-1]).max().item())

    def attention_mask(self) -> Optional[torch.Tensor]:
        """Binary [B, S] mask (1 = valid) equivalent to ``seqused`` (BSHD only)."""
        if self.layout != "bshd" or self.seqused is None:
            return None
        ar = torch.arange(self.seqlen, dtype=torch.int32)[None, :]
        return (ar < self.seqused[:, None]).to(torch.int32)


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _draw_qkv(rng, T: int):
    q = _normal(rng, (T, NUM_Q_HEADS, HEAD_DIM))
    k = _normal(rng, (T, NUM_KV_HEADS, HEAD_DIM))
    v = _normal(rng, (T, NUM_KV_HEADS, HEAD_DIM))
    return q, k, v


def _draw_params(rng, sink_std: float):
    qw = 1.0 + _normal(rng, (HEAD_DIM,), 0.1)
    kw = 1.0 + _normal(rng, (HEAD_DIM,), 0.1)
    sinks = _normal(rng, (NUM_Q_HEADS,), sink_std)
    return (torch.from_numpy(qw.astype(np.float32)), torch.from_numpy(kw.astype(np.float32)),
            torch.from_numpy(sinks.astype(np.float32)))


def _bshd(name, seed, B, S, layers, *, pad_max=0, sink_std=1.0, plus8_heads=(),
          massive_frac=0.0, explicit_positions=False, description=""):
    rng = np.random.default_rng(seed)
    pads = rng.integers(0, pad_max + 1, size=B) if pad_max > 0 else np.zeros(B, np.int64)
    T = B * S
    q, k, v = _draw_qkv(rng, T)
    qw, kw, sinks = _draw_params(rng, sink_std)
    meta = {}
    if massive_frac > 0.0:
        n_massive = int(round(massive_frac * T))
        idx = np.sort(rng.choice(T, size=n_massive, replace=False))
        v[idx] *= np.float32(1.0e3)
        meta["massive_tokens"] = idx.tolist()
    for h in plus8_heads:
        sinks[h] = 8.0
    cu = torch.arange(0, T + 1, S, dtype=torch.int32)
    seqused = torch.from_numpy((S - pads).astype(np.int32)) if pad_max > 0 else None
    positions = None
    if explicit_positions:
        positions = torch.arange(S, dtype=torch.int32).repeat(B)
    return Workload(name=name, seed=seed, layout="bshd", q=_bf16(q), k=_bf16(k), v=_bf16(v),
                    q_norm_w=qw, k_norm_w=kw, sinks=sinks, cu_seqlens=cu, seqused=seqused,
                    positions=positions, layers=list(layers), batch=B, seqlen=S,
                    description=description, meta=meta)


def _thd(name, seed, lengths_fn, layers, *, sink_std=1.0, description=""):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths_fn(rng), dtype=np.int64)
    T = int(lengths.sum())
    q, k, v = _draw_qkv(rng, T)
    qw, kw, sinks = _draw_params(rng, sink_std)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    # document-local positions: each document counts from zero
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lengths]) if T else np.zeros(0, np.int32)
    return Workload(name=name, seed=seed, layout="thd", q=_bf16(q), k=_bf16(k), v=_bf16(v),
                    q_norm_w=qw, k_norm_w=kw, sinks=sinks,
                    cu_seqlens=torch.from_numpy(cu.astype(np.int32)), seqused=None,
                    positions=torch.from_numpy(pos), layers=list(layers), description=description,
                    meta={"doc_lengths": lengths.tolist()})


CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5", "tstar")


def make_workload(name: str) -> Workload:
    """The named synthetic workloads (seed = 1000 + index, tstar = 1006)."""
    if name == "c1":
        return _bshd("c1", 1001, 1, 768, [SLIDING], explicit_positions=True,
                     description="sliding W=513 RoPE, B=1, S=768")
    if name == "c2":
        return _bshd("c2", 1002, 1, 4096, [FULL], sink_std=2.0, plus8_heads=(0, 8, 16, 24),
                     massive_frac=0.01,
                     description="full NoPE, B=1, S=4096, sinks N(0,2) with 4 heads at +8, 1% v tokens x1e3")
    if name == "c3":
        return _bshd("c3", 1003, 8, 8192, [SLIDING], pad_max=1024,
                     description="sliding W=513 RoPE, B=8, S=8192, trailing padding 0-1024")
    if name == "c4":
        return _thd("c4", 1004, lambda rng: rng.integers(128, 8193, size=16), [SLIDING, FULL],
                    description="THD 16 docs, lengths U[128,8192], document-local positions")
    if name == "c5":
        return _bshd("c5", 1005, 1, 131072, [FULL], description="full NoPE, B=1, S=131072")
    if name == "tstar":
        return _bshd("tstar", 1006, 1, 8192, [FULL], description="full NoPE, B=1, S=8192")
    raise KeyError(name)


def make_custom(seed: int, lengths: Sequence[int], *, layout: str = "thd", seqused=None,
                layers=(SLIDING,), sink_std: float = 1.0, positions: str = "local",
                q_scale: float = 1.0, norm_scale: float = 1.0, dtype: str = "bf16") -> Workload:
    """A small seeded workload for tests.

    ``lengths`` are sequence lengths (BSHD needs equal lengths). ``seqused``
    gives trailing-padding valid lengths. ``positions`` is "local" (index in the
    sequence, passed explicitly), "none" (argument left out) or "random"
    (arbitrary non-negative integers). ``norm_scale`` multiplies both RMSNorm
    weights (large weights give large logits). ``dtype`` "float32" keeps q, k, v
    as the float32 draws (the FP32 projections the FP16 attention-compute
    variant takes) instead of rounding them to bfloat16.
    """
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    q, k, v = _draw_qkv(rng, T)
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    qw, kw, sinks = _draw_params(rng, sink_std)
    if norm_scale != 1.0:
        qw = qw * np.float32(norm_scale)
        kw = kw * np.float32(norm_scale)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    if positions == "local":
        pos = torch.from_numpy(np.concatenate([np.arange(n, dtype=np.int32) for n in lengths])
                               if T else np.zeros(0, np.int32))
    elif positions == "random":
        pos = torch.from_numpy(rng.integers(0, 262144, size=T).astype(np.int32))
    else:
        pos = None
    su = None if seqused is None else torch.tensor(list(seqused), dtype=torch.int32)
    B = len(lengths) if layout == "bshd" else 0
    S = lengths[0] if layout == "bshd" and lengths else 0
    cast = _bf16 if dtype == "bf16" else (lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)))
    return Workload(name=f"custom{seed}", seed=seed, layout=layout, q=cast(q), k=cast(k),
                    v=cast(v), q_norm_w=qw, k_norm_w=kw, sinks=sinks,
                    cu_seqlens=torch.from_numpy(cu.astype(np.int32)), seqused=su, positions=pos,
                    layers=list(layers), batch=B, seqlen=S)


def make_long_decode(seed: int, n_cached: int, layers=(FULL,), sink_std: float = 1.0):
    """One sequence of n_cached + 1 tokens for a decode check at long context.

    Only the last token's query is drawn (the earlier queries never enter a
    decode step); k and v cover every token. Draw order: q of the last token,
    k, v, then weights and sinks. Returns a Workload whose q has a single row
    (the last token) and cu_seqlens = [0, 1], plus k and v for all tokens in
    ``meta["k_all"]`` / ``meta["v_all"]``.
    """
    rng = np.random.default_rng(seed)
    T = n_cached + 1
    q = _normal(rng, (1, NUM_Q_HEADS, HEAD_DIM))
    k = _normal(rng, (T, NUM_KV_HEADS, HEAD_DIM))
    v = _normal(rng, (T, NUM_KV_HEADS, HEAD_DIM))
    qw, kw, sinks = _draw_params(rng, sink_std)
    wl = Workload(name=f"longdecode{seed}", seed=seed, layout="thd", q=_bf16(q), k=_bf16(k[-1:]),
                  v=_bf16(v[-1:]), q_norm_w=qw, k_norm_w=kw, sinks=sinks,
                  cu_seqlens=torch.tensor([0, 1], dtype=torch.int32), seqused=None, positions=None,
                  layers=list(layers), description=f"one sequence, {n_cached} cached tokens")
    wl.meta["k_all"] = _bf16(k)
    wl.meta["v_all"] = _bf16(v)
    return wl



def draw_dout(seed: int, T: int, std: float = 1.0) -> torch.Tensor:
    """Upstream gradient dL/dO [T, 32, 128] for a backward check: float32
    normals (stream seeded with seed + 7919, so it is not the q/k/v stream of
    the same seed) rounded to bfloat16."""
    rng = np.random.default_rng(seed + 7919)
    return _bf16(_normal(rng, (T, NUM_Q_HEADS, HEAD_DIM), std))


def draw_block(seed: int, T: int, hidden: int = 2048):
    """Inputs of the attention block: hidden states x [T, hidden] ~ N(0, 1)
    (the block sees normalized hidden states) and the projection weights
    ~ N(0, 0.02) (FlintConfig page, initializer_range 0.02): w_q [4096, hidden],
    w_k and w_v [512, hidden], w_o [hidden, 4096]; all bf16. Returns
    (x, w_q, w_k, w_v, w_o)."""
    rng = np.random.default_rng(seed + 104729)
    x = _bf16(_normal(rng, (T, hidden)))
    w_q = _bf16(_normal(rng, (NUM_Q_HEADS * HEAD_DIM, hidden), 0.02))
    w_k = _bf16(_normal(rng, (NUM_KV_HEADS * HEAD_DIM, hidden), 0.02))
    w_v = _bf16(_normal(rng, (NUM_KV_HEADS * HEAD_DIM, hidden), 0.02))
    w_o = _bf16(_normal(rng, (hidden, NUM_Q_HEADS * HEAD_DIM), 0.02))
    return x, w_q, w_k, w_v, w_o


def draw_large(seed: int, T: int, device, chunk: int = 1 << 16):
    """q [T, 32, 128], k and v [T, 4, 128], bf16 ~ N(0, 1), drawn on `device`
    in chunks of `chunk` tokens, for sizes whose host copy would not fit; the
    same seed (and chunk) gives the same tensors. Norm weights and sinks come
    from `draw_large_params`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for heads in (NUM_Q_HEADS, NUM_KV_HEADS, NUM_KV_HEADS):
        t = torch.empty(T, heads, HEAD_DIM, dtype=torch.bfloat16, device=device)
        for a in range(0, T, chunk):
            b = min(T, a + chunk)
            t[a:b] = torch.randn(b - a, heads, HEAD_DIM, generator=g, device=device).to(torch.bfloat16)
        out.append(t)
    return tuple(out)


def draw_large_params(seed: int):
    """q_norm_w, k_norm_w ~ N(1, 0.1) [128] and sinks ~ N(0, 1) [32], float32 on the host."""
    rng = np.random.default_rng(seed + 15485863)
    qw, kw, sk = _draw_params(rng, 1.0)
    return qw, kw, sk
