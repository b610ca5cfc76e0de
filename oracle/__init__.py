"""Plain, slow fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``paged_kv_cache_254_amd``) and imports nothing from it.

Modules:

* ``kv_bytes``   - the KV-cache byte formula and its per-token / per-context
                   forms (pinned to the values the pages print).
* ``attention``  - gather through the block table, dense softmax attention per
                   (sequence, query head) with GQA/MQA head sharing, per-range
                   partials with their log-sum-exp, the log-sum-exp combine, and
                   the one-slot append (pinned to closed forms, invariants, a
                   library routine and brute force).
* ``page_pool``  - on-demand page allocation from a free list and the
                   per-request block table (pinned to its invariants and to
                   hand-worked tables).
* ``kv_quant``   - 8-bit KV cache: per-(token, KV head) uniform quantization
                   with a scale and a zero point, the quantizing append, and
                   decode over the dequantized cache (pinned to hand-worked
                   codes, exact grid round trips, the half-step bound, and the
                   decode above run on explicitly dequantized pools).

Parity status: every function here is called by at least one pin in
``tests/test_oracle_*.py``, and ``tests/test_oracle_mutations.py`` plants a
plausible mistake in each (a dropped term, a wrong index, a swapped operand,
a reversed order) and checks that one of those pins fails; none is "parity
unpinned".
"""
from . import attention, kv_bytes, kv_quant, page_pool  # noqa: F401
