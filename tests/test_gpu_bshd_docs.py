"""GPU: BSHD input with document ids and arbitrary padding.

The plan kernel's THD description is checked against one built by plain loops
here; the layer against the FP64 BSHD oracle (same bars as the bf16 parity
tests: max |err| <= 2e-2 max|V|, mean <= 1e-3 max|V|, padded rows exact
zeros); the packed path (documents with holes) against the THD path on the
same tokens packed by hand, bitwise, forward with its normalizer and backward.
"""

import numpy as np
import pytest
import torch

import attention_head_rmsnorm_amd as fa
from oracle import flint_attention, flint_attention_bshd
from workload import make_custom

from .common import f64

pytestmark = pytest.mark.gpu

MAX_FRAC = 2e-2
MEAN_FRAC = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load_library()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _dev():
    return torch.device("cuda", 0)


def expected_plan(mask, ids):
    """The THD description by loops over the tokens (see the C ABI header)."""
    B, S = mask.shape
    N = B * S
    valid = mask.reshape(-1) != 0
    idf = ids.reshape(-1)
    docs = []  # [stream start, packed start, length]
    holes = False
    prev = None
    c = 0
    for i in range(N):
        if not valid[i]:
            continue
        start = prev is None or prev // S != i // S or idf[prev] != idf[i]
        if start:
            docs.append([i, c, 0])
        elif prev != i - 1:
            holes = True
        docs[-1][2] += 1
        prev = i
        c += 1
    if holes:
        cu = [d[1] for d in docs] + [c]
        used = [d[2] for d in docs]
        return dict(n=len(docs), mx=max(used), T=c, packed=1, cu=cu, used=used)
    seqs = []
    if N and not valid[0]:
        seqs.append([0, 0])
    seqs += [[d[0], d[2]] for d in docs]
    cu = [s[0] for s in seqs] + [N]
    used = [s[1] for s in seqs]
    mx = max([cu[k + 1] - cu[k] for k in range(len(seqs))], default=0)
    return dict(n=len(seqs), mx=mx, T=N, packed=0, cu=cu, used=used)


def _mask_ids(seed, B, S, doc_lengths=None, hole_rate=0.0, lead=None, trail=None):
    rng = np.random.default_rng(seed)
    mask = np.ones((B, S), np.uint8)
    ids = np.zeros((B, S), np.int32)
    for b in range(B):
        if doc_lengths is not None:
            lens = doc_lengths[b]
            ids[b] = np.repeat(np.arange(len(lens)) + 100 * b, lens)[:S]
        if hole_rate:
            mask[b, rng.random(S) < hole_rate] = 0
        if lead is not None:
            mask[b, :lead[b]] = 0
        if trail is not None and trail[b]:
            mask[b, S - trail[b]:] = 0
    return mask, ids


CASES = [
    # name, B, S, doc lengths per row (None: one document), hole rate, lead, trail
    ("documents only", 2, 700, [[100, 1, 250, 349], [700]], 0.0, None, None),
    ("left padding", 3, 300, None, 0.0, [0, 37, 300], None),
    ("left and trailing padding, documents", 2, 400, [[150, 250], [10, 390]], 0.0, [5, 0], [0, 60]),
    ("interior holes", 2, 500, None, 0.05, None, None),
    ("holes and documents", 3, 333, [[100, 100, 133], [1, 1, 331], [333]], 0.1, [3, 0, 0], [0, 9, 0]),
    ("one-token documents", 1, 130, [[1] * 130], 0.0, None, None),
]


def _workload(seed, B, S):
    wl = make_custom(seed, [S] * B, layout="bshd")
    return wl


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_matches_loops(case):
    name, B, S, lens, rate, lead, trail = case
    mask, ids = _mask_ids(11, B, S, lens, rate, lead, trail)
    d = _dev()
    info, cu, used, pack, unpack = fa.bshd_plan(torch.from_numpy(mask).to(d),
                                                torch.from_numpy(ids).to(d), B, S, d)
    exp = expected_plan(mask, ids)
    _log(f"[gpu] plan {name}: {info[:4]} expected n={exp['n']} mx={exp['mx']} T={exp['T']} "
         f"packed={exp['packed']}")
    assert info[:4] == (exp["n"], exp["mx"], exp["T"], exp["packed"])
    assert cu.cpu().tolist() == exp["cu"]
    assert used.cpu().tolist() == exp["used"]
    if exp["packed"]:
        src = np.nonzero(mask.reshape(-1))[0]
        assert np.array_equal(pack.cpu().numpy(), src)
        inv = np.full(B * S, -1)
        inv[src] = np.arange(len(src))
        assert np.array_equal(unpack.cpu().numpy(), inv)


def test_plan_edge_shapes():
    d = _dev()
    for B, S, m in ((0, 5, None), (3, 0, None), (2, 4, np.zeros((2, 4), np.uint8)),
                    (1, 3000, None)):
        mask = None if m is None else torch.from_numpy(m).to(d)
        ids = torch.zeros((B, S), dtype=torch.int32, device=d)
        info, cu, used, _, _ = fa.bshd_plan(mask, ids, B, S, d)
        exp = expected_plan(np.ones((B, S), np.uint8) if m is None else m, np.zeros((B, S)))
        assert info[:4] == (exp["n"], exp["mx"], exp["T"], exp["packed"]), (B, S)
        assert cu.cpu().tolist() == exp["cu"] and used.cpu().tolist() == exp["used"]


def _run(wl, mask, ids, window, rope, positions=None, f16=False):
    d = _dev()
    B, S = wl.batch, wl.seqlen
    cast = (lambda t: t.float()) if f16 else (lambda t: t)
    q = cast(wl.q).to(d).view(B, S, 32, 128)
    k = cast(wl.k).to(d).view(B, S, 4, 128)
    v = cast(wl.v).to(d).view(B, S, 4, 128)
    fn = fa.flint_attn_f16 if f16 else fa.flint_attn
    return fn(q, k, v, wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d),
              attention_mask=torch.from_numpy(mask).to(d), document_ids=torch.from_numpy(ids).to(d),
              positions=None if positions is None else torch.from_numpy(positions).to(d),
              window=window, use_rope=rope)


def _grade(out, ref, wl, mask, what, max_frac=MAX_FRAC, mean_frac=MEAN_FRAC):
    got = out.float().cpu().numpy().astype(np.float64)
    ok = mask != 0
    vmax = float(np.abs(f64(wl.v)).max())
    err = np.abs(got[ok] - ref[ok])
    stats = dict(max_frac=float(err.max()) / vmax, mean_frac=float(err.mean()) / vmax)
    _log(f"      {what}: {stats}")
    assert np.all(np.isfinite(got)), what
    assert stats["max_frac"] <= max_frac and stats["mean_frac"] <= mean_frac, (what, stats)
    assert np.all(got[~ok] == 0.0), f"{what}: padded rows are not zeros"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_parity_with_oracle(case):
    name, B, S, lens, rate, lead, trail = case
    mask, ids = _mask_ids(12, B, S, lens, rate, lead, trail)
    wl = _workload(400 + len(name), B, S)
    _log(f"[gpu] BSHD documents parity: {name} B={B} S={S}")
    for window, rope in ((513, True), (0, False), (33, True)):
        out = _run(wl, mask, ids, window, rope)
        torch.cuda.synchronize()
        ref = flint_attention_bshd(f64(wl.q).reshape(B, S, 32, 128), f64(wl.k).reshape(B, S, 4, 128),
                                   f64(wl.v).reshape(B, S, 4, 128), f64(wl.q_norm_w),
                                   f64(wl.k_norm_w), f64(wl.sinks), attention_mask=mask,
                                   document_ids=ids, window=window, use_rope=rope)
        _grade(out, ref, wl, mask, f"{name} w={window}")


def test_explicit_positions_with_holes():
    B, S = 2, 400
    mask, ids = _mask_ids(13, B, S, [[200, 200], [400]], 0.08)
    pos = np.random.default_rng(13).integers(0, 100000, (B, S)).astype(np.int32)
    wl = _workload(431, B, S)
    out = _run(wl, mask, ids, 513, True, positions=pos)
    torch.cuda.synchronize()
    ref = flint_attention_bshd(f64(wl.q).reshape(B, S, 32, 128), f64(wl.k).reshape(B, S, 4, 128),
                               f64(wl.v).reshape(B, S, 4, 128), f64(wl.q_norm_w), f64(wl.k_norm_w),
                               f64(wl.sinks), attention_mask=mask, document_ids=ids,
                               position_ids=pos, window=513, use_rope=True)
    _grade(out, ref, wl, mask, "explicit positions")


def test_fp16_variant_with_holes():
    B, S = 2, 300
    mask, ids = _mask_ids(14, B, S, [[100, 200], [300]], 0.1, lead=[4, 0])
    wl = make_custom(432, [S] * B, layout="bshd", dtype="float32")
    out = _run(wl, mask, ids, 513, True, f16=True)
    torch.cuda.synchronize()
    ref = flint_attention_bshd(f64(wl.q).reshape(B, S, 32, 128), f64(wl.k).reshape(B, S, 4, 128),
                               f64(wl.v).reshape(B, S, 4, 128), f64(wl.q_norm_w), f64(wl.k_norm_w),
                               f64(wl.sinks), attention_mask=mask, document_ids=ids, window=513,
                               use_rope=True)
    _grade(out, ref, wl, mask, "fp16 holes", max_frac=4e-3, mean_frac=2.5e-4)


def _hand_packed(wl, mask, ids):
    """THD tensors of the valid tokens in order, cut at document runs (numpy)."""
    B, S = mask.shape
    src = np.nonzero(mask.reshape(-1))[0]
    idf = ids.reshape(-1)
    lengths = []
    for j, i in enumerate(src):
        if j == 0 or src[j - 1] // S != i // S or idf[src[j - 1]] != idf[i]:
            lengths.append(0)
        lengths[-1] += 1
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return src, cu


def test_packed_path_equals_thd_bitwise_forward_and_backward():
    B, S = 2, 600
    mask, ids = _mask_ids(15, B, S, [[300, 50, 250], [600]], 0.07, lead=[0, 11], trail=[13, 0])
    wl = _workload(433, B, S)
    d = _dev()
    src, cu = _hand_packed(wl, mask, ids)
    si = torch.from_numpy(src).to(d)
    q = wl.q.to(d).view(B, S, 32, 128)
    k = wl.k.to(d).view(B, S, 4, 128)
    v = wl.v.to(d).view(B, S, 4, 128)
    w = (wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d))
    m_t, i_t = torch.from_numpy(mask).to(d), torch.from_numpy(ids).to(d)
    from workload.gen import draw_dout
    dout = draw_dout(433, B * S).to(d).view(B, S, 32, 128)
    for window in (513, 0):
        kw = dict(window=window, use_rope=window > 0)
        out, lse = fa.flint_attn(q, k, v, *w, attention_mask=m_t, document_ids=i_t,
                                 return_lse=True, **kw)
        grads = fa.flint_attn_backward(dout, q, k, v, *w, out, lse, attention_mask=m_t,
                                       document_ids=i_t, **kw)
        qt, kt, vt = (x.reshape(B * S, *x.shape[2:])[si].contiguous() for x in (q, k, v))
        cu_t = torch.from_numpy(cu).to(d)
        o2, l2 = fa.flint_attn(qt, kt, vt, *w, cu_seqlens=cu_t, return_lse=True, **kw)
        g2 = fa.flint_attn_backward(dout.reshape(B * S, 32, 128)[si].contiguous(), qt, kt, vt, *w,
                                    o2, l2, cu_seqlens=cu_t, **kw)
        torch.cuda.synchronize()
        flat = lambda x: x.reshape(B * S, *x.shape[2:])  # noqa: E731
        assert torch.equal(flat(out)[si], o2), f"forward w={window}"
        assert torch.equal(flat(lse)[si], l2), f"lse w={window}"
        pad = torch.from_numpy(mask.reshape(-1) == 0).to(d)
        assert torch.all(flat(out)[pad] == 0) and torch.all(torch.isneginf(flat(lse)[pad]))
        for name, a, b in zip(("dq", "dk", "dv"), grads[:3], g2[:3]):
            assert torch.equal(flat(a)[si], b), f"{name} w={window}"
            assert torch.all(flat(a)[pad] == 0), f"{name} padded rows w={window}"
        for name, a, b in zip(("dq_norm_w", "dk_norm_w", "dsinks"), grads[3:], g2[3:]):
            assert torch.equal(a, b), f"{name} w={window}"


def test_documents_in_place_equal_thd_bitwise():
    """Without holes the BSHD buffers are used in place: the same as THD with
    the document boundaries (and trailing padding as seqused)."""
    B, S = 2, 512
    mask, ids = _mask_ids(16, B, S, [[100, 412], [256, 256]], 0.0, trail=[12, 0])
    wl = _workload(434, B, S)
    d = _dev()
    q = wl.q.to(d).view(B, S, 32, 128)
    k = wl.k.to(d).view(B, S, 4, 128)
    v = wl.v.to(d).view(B, S, 4, 128)
    w = (wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d))
    a = fa.flint_attn(q, k, v, *w, attention_mask=torch.from_numpy(mask).to(d),
                      document_ids=torch.from_numpy(ids).to(d))
    cu = torch.tensor([0, 100, 512, 768, 1024], dtype=torch.int32, device=d)
    su = torch.tensor([100, 400, 256, 256], dtype=torch.int32, device=d)
    b = fa.flint_attn(q.view(B * S, 32, 128), k.view(B * S, 4, 128), v.view(B * S, 4, 128), *w,
                      cu_seqlens=cu, seqused=su, max_seqlen=412)
    torch.cuda.synchronize()
    assert torch.equal(a.view(B * S, 32, 128), b)


def test_long_packed_rows_sampled():
    """4 rows of 8,192 tokens holding documents of mixed lengths (log-uniform
    64..4096) with 2% holes: the packed path equals THD on the hand-packed
    tokens bitwise, and sampled rows match the THD oracle."""
    B, S = 4, 8192
    rng = np.random.default_rng(17)
    lens = []
    for _ in range(B):
        row, left = [], S
        while left > 0:
            n = int(min(left, np.exp(rng.uniform(np.log(64), np.log(4096)))))
            row.append(n)
            left -= n
        lens.append(row)
    mask, ids = _mask_ids(17, B, S, lens, 0.02)
    wl = _workload(435, B, S)
    d = _dev()
    src, cu = _hand_packed(wl, mask, ids)
    si = torch.from_numpy(src).to(d)
    q = wl.q.to(d).view(B, S, 32, 128)
    k = wl.k.to(d).view(B, S, 4, 128)
    v = wl.v.to(d).view(B, S, 4, 128)
    w = (wl.q_norm_w.to(d), wl.k_norm_w.to(d), wl.sinks.to(d))
    _log(f"[gpu] long packed rows: {sum(len(x) for x in lens)} documents, {len(src)} valid tokens")
    out = fa.flint_attn(q, k, v, *w, attention_mask=torch.from_numpy(mask).to(d),
                        document_ids=torch.from_numpy(ids).to(d))
    qt, kt, vt = (x.reshape(B * S, *x.shape[2:])[si].contiguous() for x in (q, k, v))
    o2 = fa.flint_attn(qt, kt, vt, *w, cu_seqlens=torch.from_numpy(cu).to(d))
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(B * S, 32, 128)[si], o2)
    rows = np.unique(np.concatenate([cu[:-1][:40], rng.integers(0, len(src), 200)]))
    ref = flint_attention(f64(wl.q)[src], f64(wl.k)[src], f64(wl.v)[src], f64(wl.q_norm_w),
                          f64(wl.k_norm_w), f64(wl.sinks), cu.astype(np.int64), window=513,
                          use_rope=True, rows=rows)
    got = o2[torch.from_numpy(rows).to(d)].float().cpu().numpy().astype(np.float64)
    vmax = float(np.abs(f64(wl.v)).max())
    err = np.abs(got - ref)
    _log(f"      sampled rows {len(rows)}: max_frac {err.max() / vmax:.3g} mean_frac {err.mean() / vmax:.3g}")
    assert err.max() <= MAX_FRAC * vmax and err.mean() <= MEAN_FRAC * vmax


@pytest.mark.parametrize("holes", [False, True])
def test_plan_many_blocks(holes):
    """More than 1,024 blocks of tokens (each phase sums over earlier blocks in strides)."""
    B, S = 130, 8192
    rng = np.random.default_rng(18)
    ids = np.cumsum(rng.random((B, S)) < 1e-3, axis=1).astype(np.int32)
    mask = np.ones((B, S), np.uint8)
    mask[rng.random((B, S)) < (0.01 if holes else 0.0)] = 0
    mask[:, -5:] = 0
    d = _dev()
    info, cu, used, pack, unpack = fa.bshd_plan(torch.from_numpy(mask).to(d),
                                                torch.from_numpy(ids).to(d), B, S, d)
    exp = expected_plan(mask, ids)
    _log(f"[gpu] plan {B}x{S} holes={holes}: {info[:4]}")
    assert info[:4] == (exp["n"], exp["mx"], exp["T"], exp["packed"])
    assert np.array_equal(cu.cpu().numpy(), np.array(exp["cu"]))
    assert np.array_equal(used.cpu().numpy(), np.array(exp["used"]))
