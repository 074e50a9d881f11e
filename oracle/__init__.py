"""CPU oracle for block-sparse attention prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The library's product path never routes through it, and it shares no
code with the HIP kernels: it imports nothing from ``block_sparse_attention_36_amd``
and nothing from ``workloads``.  See ``oracle/bsa_oracle.py`` for the method,
written out step by step in float64 NumPy.
"""

from .bsa_oracle import *  # noqa: F401,F403
