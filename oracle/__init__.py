"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition that the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The library under
``exact_attention_20_amd/`` never imports it, and it never imports that
library: the two share no code. Inputs come from ``workloads`` (seeded random
numbers only).

Every function is written in numpy float64 from the pages' statement of the
method (citations per function). Pins that tie it to facts other than itself
live in ``tests/test_oracle_pins.py``; none of its functions is unpinned.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    attention_head,
    attention_head_backward,
    causal_allowed,
    e4m3fn_to_float,
    gather_pages,
    kv_append,
    kv_head_of,
    lse_merge,
    paged_decode,
    paged_prefill,
    paged_prefill_request,
    prefill,
    prefill_backward,
    scores,
    softmax_rows,
)
