"""fp64 CPU oracle of the MoDA joint sequence/depth attention (forward, decode, backward).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline leg may import it. It shares no code with the HIP library."""
from .moda_oracle import (  # noqa: F401
    decode,
    depth_kv_projection,
    depth_only,
    depth_utilization,
    depth_visible,
    expanded_rows_attention,
    joint_attention,
    joint_attention_backward,
    joint_rows,
    scalar_ref,
    select_slots,
    separate_then_add,
    sequence_only,
    sequence_visible,
)
