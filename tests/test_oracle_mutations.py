"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

Every mutation swaps one oracle function for a wrong variant, then runs the
pins; the test passes when at least one pin fails. This shows that the pins
pin the oracle down: a dropped term, a wrong sign, index or operand anywhere in
it is seen.
"""

import math

import numpy as np
import pytest

import oracle.flint_oracle as fo

from . import oracle_pins

_rms = fo.rms_norm
_rope = fo.rope_neox
_freq = fo.rope_frequencies
_allowed = fo.allowed_keys
_softmax = fo.sink_softmax
_kv = fo.kv_head_of


def _rms_one_plus_w(x, w, eps):
    return _rms(x, 1.0 + np.asarray(w, np.float64), eps)


def _rms_eps_outside(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * w


def _rms_no_weight(x, w, eps):
    return _rms(x, np.ones_like(np.asarray(w, np.float64)), eps)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    perm = np.concatenate([np.arange(0, x.shape[-1], 2), np.arange(1, x.shape[-1], 2)])
    inv = np.argsort(perm)
    return _rope(x[..., perm], pos, theta)[..., inv]


def _freq_half_rate(head_dim, theta):
    c = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -c / head_dim)


def _rope_reversed(x, pos, theta):
    return _rope(x, -np.asarray(pos, np.float64), theta)


def _rope_position_plus_one(x, pos, theta):
    return _rope(x, np.asarray(pos, np.float64) + 1, theta)


def _window_off_by_one(lq, lk, valid_len, window):
    return _allowed(lq, lk, valid_len, window + 1 if window > 0 else 0)


def _non_causal_by_one(lq, lk, valid_len, window):
    return _allowed(np.asarray(lq) + 1, lk, valid_len, window)


def _sink_scaled(z, sink):
    return _softmax(z, np.asarray(sink, np.float64) / math.sqrt(128))


def _sink_dropped(z, sink):
    w, _, m, e = _softmax(z, np.full_like(np.asarray(sink, np.float64), -np.inf))
    return w, np.zeros_like(np.asarray(m)), m, e


def _sink_as_zero_logit_token(z, sink):
    return _softmax(z, np.zeros_like(np.asarray(sink, np.float64)))


def _logits_unscaled(z, sink):
    return _softmax(z * math.sqrt(128), sink)


def _gqa_modulo(h, num_q_heads, num_kv_heads):
    return h % num_kv_heads


MUTATIONS = {
    "rmsnorm 1+w": ("rms_norm", _rms_one_plus_w),
    "rmsnorm eps outside sqrt": ("rms_norm", _rms_eps_outside),
    "rmsnorm weight dropped": ("rms_norm", _rms_no_weight),
    "rope interleaved pairs": ("rope_neox", _rope_interleaved),
    "rope frequencies half rate": ("rope_frequencies", _freq_half_rate),
    "rope rotation sign": ("rope_neox", _rope_reversed),
    "rope position off by one": ("rope_neox", _rope_position_plus_one),
    "window 514": ("allowed_keys", _window_off_by_one),
    "causal off by one": ("allowed_keys", _non_causal_by_one),
    "sink scaled by 1/sqrt(d)": ("sink_softmax", _sink_scaled),
    "sink dropped": ("sink_softmax", _sink_dropped),
    "sink as zero-logit token": ("sink_softmax", _sink_as_zero_logit_token),
    "logits unscaled": ("sink_softmax", _logits_unscaled),
    "gqa h % 4": ("kv_head_of", _gqa_modulo),
}

# Keeping padded keys is not a mutation here: padding is trailing, so every
# padded key lies after every valid query and causality already drops it.

# cheap pins first: the first failure ends the run for that mutation
_ORDER = sorted(oracle_pins.ALL_PINS, key=lambda f: (f.__name__ in (
    "pin_window_count", "pin_rope_frequencies_library", "pin_library_layer"), f.__name__))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(fo, attr, bad)
    caught = []
    for pin in _ORDER:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake '{name}'"


# ---------------------------------------------------------------- backward oracle

import oracle.flint_oracle_bwd as fb  # noqa: E402

from . import oracle_bwd_pins  # noqa: E402

_rope_adj = fb._rope_adjoint
_rms_bwd = fb._rms_norm_backward
_sm_bwd = fb._softmax_backward


def _rope_adjoint_forward_turn(x, pos, theta):
    return fo.rope_neox(x, pos, theta)


def _rms_bwd_no_mean_term(x, w, eps, dy):
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return r * dy * w, dy * x * r


def _rms_bwd_weight_unnormalized(x, w, eps, dy):
    dx, _ = _rms_bwd(x, w, eps, dy)
    return dx, dy * np.asarray(x, np.float64)


def _rms_bwd_weight_missing(x, w, eps, dy):
    return _rms_bwd(x, np.ones_like(np.asarray(w, np.float64)), eps, dy)


def _softmax_bwd_no_row_term(W, dW, Dr):
    return W * dW


def _softmax_bwd_row_term_unweighted(W, dW, Dr):
    return W * dW - Dr[:, None]


def _sink_adjoint_sign(p, Dr):
    return float(np.sum(p * Dr))


def _sink_adjoint_complement(p, Dr):
    return -float(np.sum((1.0 - p) * Dr))


BWD_MUTATIONS = {
    "rope adjoint turns forward": ("_rope_adjoint", _rope_adjoint_forward_turn),
    "rmsnorm backward without the mean term": ("_rms_norm_backward", _rms_bwd_no_mean_term),
    "norm weight gradient unnormalized": ("_rms_norm_backward", _rms_bwd_weight_unnormalized),
    "norm weight missing in backward": ("_rms_norm_backward", _rms_bwd_weight_missing),
    "softmax backward without Dr": ("_softmax_backward", _softmax_bwd_no_row_term),
    "softmax backward Dr not weighted": ("_softmax_backward", _softmax_bwd_row_term_unweighted),
    "sink adjoint sign": ("_sink_adjoint", _sink_adjoint_sign),
    "sink adjoint with 1 - p": ("_sink_adjoint", _sink_adjoint_complement),
    "logit scale 1": ("_logit_scale", lambda d: 1.0),
}

_BWD_ORDER = list(oracle_bwd_pins.ALL_PINS)  # already cheapest first


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_mutation_is_caught(name, monkeypatch):
    attr, bad = BWD_MUTATIONS[name]
    monkeypatch.setattr(fb, attr, bad)
    caught = []
    for pin in _BWD_ORDER:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no backward pin caught the planted mistake '{name}'"


# ----------------------------------------------------------------- BSHD documents and padding

import oracle.flint_oracle_bshd as fd  # noqa: E402

from . import oracle_bshd_pins  # noqa: E402

_doc_structure = fd.document_structure
_doc_allowed = fd._allowed


def _allowed_window_in_columns(rank, doc, window):
    cols = np.where(rank >= 0, np.arange(len(rank)), -1)
    ok = _doc_allowed(rank, doc, 0)
    if window > 0:
        ok &= (cols[:, None] - cols[None, :]) <= (window - 1)
    return ok


def _allowed_window_off_by_one(rank, doc, window):
    return _doc_allowed(rank, doc, window + 1 if window > 0 else 0)


def _allowed_not_causal(rank, doc, window):
    ok = _doc_allowed(rank, doc, 0) | _doc_allowed(rank, doc, 0).T
    if window > 0:
        ok &= np.abs(rank[:, None] - rank[None, :]) <= (window - 1)
    return ok


def _docs_by_id(valid, ids):
    rank, doc, local = _doc_structure(valid, ids)
    doc = np.where(doc >= 0, np.asarray(ids, np.int64), -1)
    for s in range(len(valid)):
        if doc[s] >= 0:
            local[s] = int(np.sum(doc[:s] == doc[s]))
    return rank, doc, local


def _positions_are_columns(valid, ids):
    # (counting from the row's first valid token instead of the document's is
    # no mistake: RoPE logits see position differences only)
    rank, doc, _ = _doc_structure(valid, ids)
    return rank, doc, np.where(rank >= 0, np.arange(len(rank)), -1)


def _padding_splits_documents(valid, ids):
    S = len(valid)
    rank, doc, local = _doc_structure(valid, ids)
    d = -1
    start = 0
    for s in range(S):
        if not valid[s]:
            continue
        if s == 0 or not valid[s - 1] or ids[s] != ids[s - 1]:
            d += 1
            start = rank[s]
        doc[s] = d
        local[s] = rank[s] - start
    return rank, doc, local


BSHD_MUTATIONS = {
    "window counts columns": ("_allowed", _allowed_window_in_columns),
    "window off by one": ("_allowed", _allowed_window_off_by_one),
    "not causal": ("_allowed", _allowed_not_causal),
    "documents by id equality": ("document_structure", _docs_by_id),
    "default positions are row columns": ("document_structure", _positions_are_columns),
    "padding splits a document": ("document_structure", _padding_splits_documents),
}


@pytest.mark.parametrize("name", sorted(BSHD_MUTATIONS))
def test_bshd_mutation_is_caught(name, monkeypatch):
    attr, bad = BSHD_MUTATIONS[name]
    monkeypatch.setattr(fd, attr, bad)
    caught = []
    for pin in oracle_bshd_pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no BSHD pin caught the planted mistake '{name}'"


# ----------------------------------------------------------------- attention block

import oracle.flint_oracle_block as fblk  # noqa: E402

from . import oracle_block_pins  # noqa: E402

_linear = fblk.linear
_split = fblk.split_heads


def _split_dim_major(y, head_dim):
    T = y.shape[0]
    return y.reshape(T, head_dim, y.shape[1] // head_dim).transpose(0, 2, 1)


def _linear_plus_bias(x, w):
    return _linear(x, w) + 0.01


def _linear_weight_transposed_blocks(x, w):
    # rows of W taken in reversed order: the output channels come out reversed
    return _linear(x, np.asarray(w)[::-1])


BLOCK_MUTATIONS = {
    "heads split dim-major": ("split_heads", _split_dim_major),
    "projection with a bias": ("linear", _linear_plus_bias),
    "output channels reversed": ("linear", _linear_weight_transposed_blocks),
}


@pytest.mark.parametrize("name", sorted(BLOCK_MUTATIONS))
def test_block_mutation_is_caught(name, monkeypatch):
    attr, bad = BLOCK_MUTATIONS[name]
    monkeypatch.setattr(fblk, attr, bad)
    caught = []
    for pin in oracle_block_pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no block pin caught the planted mistake '{name}'"
