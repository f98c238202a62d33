"""fp64 CPU oracle for attention, its JVP and its reverse-mode derivative --
test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The GPU product path never
imports it and shares no code with it.
"""

from .attention_jvp import (attention, attention_jvp, attention_jvp_rows, attention_vjp,
                            attention_vjp_keys, ROW_CHUNK)

__all__ = ["attention", "attention_jvp", "attention_jvp_rows", "attention_vjp",
           "attention_vjp_keys", "ROW_CHUNK"]
