"""CPU oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path.
"""
from .attention import (attention_backward_cols, attention_backward_reference, attention_backward_rows,
                        attention_online, attention_probabilities, attention_reference)

__all__ = ["attention_reference", "attention_online", "attention_probabilities", "attention_backward_reference",
           "attention_backward_rows", "attention_backward_cols"]
