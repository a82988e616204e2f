"""fp64 CPU oracle of the sink-routed decode path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library never does.  Parity-pinned functions are listed in
``sinkrouter``'s module docstring; none is unpinned.
"""
from .sinkrouter import (  # noqa: F401
    attend_group, bos_mass, cosine, default_scale, dense_decode, group_mask, merge_partials,
    oracle_sink_events, proxy_precision_recall, record_sink, rope, rope_append, round_bf16,
    route, route_scores,
    routed_decode, split_k_decode, split_partials, threshold_sweep,
    work_list,
)
