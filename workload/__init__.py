"""Seeded synthetic inputs for the Flint sink-attention prefill layer.

This package only draws random inputs and their structure (sequence lengths,
padding, positions). It holds none of the layer's arithmetic, so both the FP64
oracle and the HIP path can take their inputs from it without sharing any of
the computation.
"""

from .gen import (  # noqa: F401
    CONFIG_NAMES,
    Layer,
    Workload,
    make_workload,
    make_custom,
    make_long_decode,
    draw_block,
    draw_dout,
    draw_large,
    draw_large_params,
)
