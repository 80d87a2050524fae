"""Seeded synthetic inputs for the lightning-indexer step.

This package only draws and quantises input tensors.  It holds none of the
indexer's arithmetic (no scoring, no visibility rule, no selection), so both
the HIP path and the CPU oracle can read the same bytes from it without
sharing any of the method's code.
"""

from .gen import CONFIGS, IndexerInputs, generate, config_names  # noqa: F401
