"""CPU oracle of the teacher-record check (test infrastructure).

TEST INFRASTRUCTURE ONLY.  This module may be imported, called or executed by
``tests/`` -- nothing else.  The HIP library and its Python binding never
import it, and it imports nothing from them.

What it computes
----------------
The cached teacher record lists, per position, the K most probable teacher
tokens (agentlenshq.com page "LLMのための効率的な知識蒸留…", section
"1. Top-K Logit Cachingによるオフライン蒸留"), so a valid row holds K distinct
ids of the vocabulary [0, v).  Over the unmasked rows (all rows when no mask
is given) it reports how many rows hold an id outside [0, v), how many hold an
id more than once, and the first row of each kind (-1 when there is none).
Masked rows are not looked at.  Plain Python per row: a range test on each id
and a set of the row's ids.
"""
from __future__ import annotations

import numpy as np


def validate_teacher(ids, v: int, mask=None):
    """ids: int [n, k]; mask: [n] (0 = skip) or None.  Returns
    (rows_out_of_range, rows_repeated, first_out_of_range, first_repeated)."""
    ids = np.asarray(ids)
    n = ids.shape[0]
    n_range = n_rep = 0
    first_range = first_rep = -1
    for i in range(n):
        if mask is not None and int(mask[i]) == 0:
            continue
        row = [int(x) for x in ids[i]]
        if any(x < 0 or x >= v for x in row):
            n_range += 1
            if first_range < 0:
                first_range = i
        if len(set(row)) < len(row):
            n_rep += 1
            if first_rep < 0:
                first_rep = i
    return n_range, n_rep, first_range, first_rep
