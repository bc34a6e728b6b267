"""CPU oracle of the W4A4 quantized linear layer — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package.  The library (w4a4_post_quantized_amd) never
imports it and shares no code with it.  See w4a4_oracle.py for the steps and
the passages of the pages each one follows.

kv_oracle.py is the INT4 KV cache with per-head transforms and the decode
attention over it (pinned by tests/test_kv_oracle_pins.py); ternary_oracle.py
is the ternary-weight layer of PT2-LLM with its ITF fitting (pinned by
tests/test_ternary_oracle_pins.py).

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against brute force, closed forms, hand-computed values (tests/golden/) or
library routines computing the same quantity another way.  The pages print no
worked numerical example of the layer and no accuracy number that could be
reproduced without trained weights and datasets, so end-to-end model accuracy
is "parity unpinned" (and out of scope).
"""
from .w4a4_oracle import *  # noqa: F401,F403
from . import kv_oracle  # noqa: F401
from . import ternary_oracle  # noqa: F401
