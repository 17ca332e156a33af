"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code, header, helper or constant with the HIP library; the only thing
both sides use is the seeded input generator in ``workloads``, which holds none
of the method's arithmetic.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed forms,
invariants, special cases and a library routine; none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention,
    attention_rows,
    attention_varlen,
    decode,
    decode_paged,
    decode_q4,
    decode_q4_paged,
    dequantize_e2m1_rows,
    quantize_e2m1_rows,
    e2m1_value,
    hadamard,
    gather_pages,
    merge_pair,
    merge_partials,
    online_softmax_tiled,
    softmax_probabilities,
    split_partials,
    empty_partial,
    fp16_exp_overflow_threshold,
    kv_head_of,
)
