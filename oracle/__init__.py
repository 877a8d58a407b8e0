"""CPU oracle for attention with per-head learnable sinks.

TEST INFRASTRUCTURE ONLY. This package exists to check the HIP path. Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import it. The library under ``attention_learnable_sinks_amd`` never
imports it, and it never imports that library: the two share no code.

Everything is plain float64 numpy that follows the method as the pages state
it; see ``oracle/sink_attention.py`` for the citations.
"""

from .sink_attention import (  # noqa: F401
    visible_mask,
    sink_attention_forward,
    sink_attention_backward,
    visible_pairs,
)
