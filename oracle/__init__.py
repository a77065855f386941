"""CPU fp64 oracle for absorbed-MLA decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and the library never calls it.
"""
from .mla_oracle import (  # noqa: F401
    bf16_to_f64,
    e4m3_to_f64,
    cache_values,
    gather,
    reconstruct_kv,
    visible_limit,
    attend,
    absorb_q,
    absorbed_scores,
    decode,
    decode_one,
    partial,
    combine,
    up_v,
    prefill,
)
from .append_oracle import (  # noqa: F401
    rope,
    f64_to_bf16_bits,
    f64_to_e4m3_bits,
    append_positions,
    append_values,
    encode_records,
    apply_append,
    with_appended,
)
from .tpla_oracle import (  # noqa: F401
    hadamard,
    rotated,
    shard_channels,
    aggregate,
    tpla_decode,
)
from .gqla_oracle import (  # noqa: F401
    group_of,
    gqa_stream,
    gqa_decode,
)
