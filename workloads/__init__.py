"""Seeded synthetic inputs (no method arithmetic) for tests and the benchmark."""
from .synth import (  # noqa: F401
    CONFIGS, L70B_128K_B8, L8B_128K, L8B_256K_B4, L8B_512K, SINK_FRACTIONS, TINY,
    Layer, Workload, as_numpy, make_caches, make_caches_device, make_k0, make_layer,
    make_layer_bulk, make_queries,
    planted_sinks, rope_inv_freq, sweep,
)
