"""fp64 CPU oracle (test infrastructure only; see kd_oracle.py).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .kd_oracle import (  # noqa: F401
    widen, teacher_distribution, student_logits, row_logsumexp,
    kd_forward, kd_backward, widen_inputs, run, dw_vocab_rows,
)
from .topk import teacher_topk  # noqa: F401
from .validate import validate_teacher  # noqa: F401
