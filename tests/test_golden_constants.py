"""The oracle and the generators against the constants the pages print."""

import json
import os

import numpy as np

from workload import make_custom
from workload.gen import HEAD_DIM, NUM_KV_HEADS, NUM_Q_HEADS, RMS_EPS, SLIDING, SLIDING_WINDOW

from .common import oracle_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flint_layer_constants.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def test_layout_constants():
    g = _g()
    assert NUM_Q_HEADS == g["num_attention_heads"]["value"]
    assert NUM_KV_HEADS == g["num_key_value_heads"]["value"]
    assert HEAD_DIM == g["head_dim"]["value"]
    assert SLIDING_WINDOW == g["sliding_window"]["value"]
    assert RMS_EPS == g["rms_norm_eps"]["value"]


def test_layer_schedule_counts():
    g = _g()["full_attention_layers"]
    full = g["value"]
    assert len(full) == g["count"] == 14
    assert 49 - len(full) == 35
    # "0, 1, 5, 9, ..., 45, and 48": every fourth layer from 1, plus 0 and 48
    assert full == [0] + list(range(1, 46, 4)) + [48]


def test_oracle_window_holds_513_keys():
    """A query deep in a sliding layer sees exactly the printed number of keys."""
    n_keys = _g()["keys_in_full_window"]["value"]
    wl = make_custom(7, [n_keys + 40], q_scale=0.0)
    _, dbg = oracle_for(wl, SLIDING, debug=True)
    counts = (dbg["weights"][:, 3, :] > 0).sum(-1)
    assert counts.max() == n_keys
    assert np.all(counts[n_keys - 1:] == n_keys)
