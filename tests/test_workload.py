"""The seeded generators: reproducible, and shaped like the named workloads."""

import hashlib

import numpy as np
import torch

from workload import make_custom, make_workload


def _digest(wl):
    h = hashlib.sha256()
    for t in (wl.q, wl.k, wl.v):
        h.update(t.view(torch.int16).numpy().tobytes())
    for t in (wl.q_norm_w, wl.k_norm_w, wl.sinks, wl.cu_seqlens):
        h.update(t.numpy().tobytes())
    return h.hexdigest()


def test_seed_reproducible():
    assert _digest(make_workload("c1")) == _digest(make_workload("c1"))
    assert _digest(make_custom(5, [30, 7], layout="thd")) == _digest(make_custom(5, [30, 7], layout="thd"))
    assert _digest(make_custom(5, [30, 7], layout="thd")) != _digest(make_custom(6, [30, 7], layout="thd"))


def test_c1_shape():
    wl = make_workload("c1")
    assert wl.q.shape == (768, 32, 128) and wl.q.dtype == torch.bfloat16
    assert wl.k.shape == (768, 4, 128) and wl.v.shape == (768, 4, 128)
    assert wl.sinks.dtype == torch.float32 and wl.sinks.shape == (32,)
    assert wl.layers[0].window == 513 and wl.layers[0].use_rope
    assert torch.equal(wl.positions, torch.arange(768, dtype=torch.int32))
    w = wl.q_norm_w.numpy()
    assert abs(w.mean() - 1.0) < 0.05 and 0.05 < w.std() < 0.15


def test_c2_structure():
    wl = make_workload("c2")
    assert wl.layers[0].window == 0 and not wl.layers[0].use_rope
    s = wl.sinks.numpy()
    assert np.all(s[[0, 8, 16, 24]] == 8.0)
    idx = wl.meta["massive_tokens"]
    assert len(idx) == 41
    big = wl.v.float().abs().amax(dim=(1, 2)).numpy()
    assert np.all(big[idx] > 100.0)
    rest = np.setdiff1d(np.arange(4096), idx)
    assert np.all(big[rest] < 10.0)


def test_c4_structure():
    wl = make_workload("c4")
    lens = np.diff(wl.cu_seqlens.numpy())
    assert len(lens) == 16 and lens.min() >= 128 and lens.max() <= 8192
    assert wl.q.shape[0] == lens.sum()
    pos = wl.positions.numpy()
    cu = wl.cu_seqlens.numpy()
    for d in range(16):
        assert np.array_equal(pos[cu[d]:cu[d + 1]], np.arange(lens[d]))
    assert [l.window for l in wl.layers] == [513, 0]


def test_bshd_padding_mask():
    wl = make_custom(9, [10, 10], layout="bshd", seqused=[4, 10])
    m = wl.attention_mask()
    assert m.shape == (2, 10)
    assert m[0].tolist() == [1] * 4 + [0] * 6 and m[1].tolist() == [1] * 10
