"""CPU oracle for exact attention forward, its gradients and KV-cache decode (TEST INFRASTRUCTURE).

Plain, slow, float64 NumPy code that materialises the full score matrix. It is
the yardstick the HIP kernels are checked against and is never part of the
product path: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it. It shares no code with the GPU library;
both sides draw their inputs from ``attn_inputs`` only.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, invariants, a pure-Python brute force and hand-worked fixtures;
the gradients against central finite differences of the forward.
No page prints numeric attention outputs, so beyond those pins the large
random configurations are pinned only through this oracle.
"""
from .exact import (  # noqa: F401
    as_fp32_scale, scores, visibility, softmax_rows, attention_head, attention,
    attention_rows, attention_varlen, decode, decode_paged,
)
from .blockwise import blockwise_attention_head, merge_partials  # noqa: F401
from .backward import attention_head_bwd, attention_bwd  # noqa: F401
