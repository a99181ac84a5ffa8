"""fp64 CPU oracle of the KDA core.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg, never by the library.  It shares no code, header,
table or helper with the HIP path.

* `gate`, `prefill`, `decode` call the plain C recurrence in kda_oracle.c
  (token by token, fp64); `prefill_backward` is its reverse-mode gradient,
  step by step through the same recurrence, and `gate_backward` the gate's.
* `chunked.prefill_chunked` is an independent fp64 chunked form used only to
  pin the recurrence (the two must agree for every chunk size).
* `prologue.shortconv_l2norm` is the layer's prologue (short causal conv,
  SiLU, q/k L2 norm), plain numpy per sequence.

Every function is pinned by a CPU test (closed forms, special cases, brute
force, the audit page's printed exp(A_log) statistics; the backward against
central differences, torch autograd and a closed form); none is "parity
unpinned".
"""
from .api import (gate, gate_backward, prefill, prefill_backward, decode,  # noqa: F401
                  build_oracle, oracle_lib_path)
from .prologue import shortconv_l2norm  # noqa: F401
