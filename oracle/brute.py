"""Loop-by-loop contiguous attention for tiny inputs (no block table, no numpy kernels).

TEST INFRASTRUCTURE ONLY: used to pin the paged oracle on tiny cases.  It works on each
sequence's logical K/V rows as plain Python lists, so it exercises none of the paging code.
The formula is textbook scaled dot-product attention with a max-shifted softmax; keys
0 .. visible-1 are seen (cloudmash "Batching and PagedAttention", "PagedAttention" step 4).
"""
from __future__ import annotations

import math
from typing import List, Sequence


def attention_row(q: Sequence[float], keys: Sequence[Sequence[float]],
                  values: Sequence[Sequence[float]], scale: float, visible: int) -> List[float]:
    """Attention of one query over the first ``visible`` key/value rows, in Python floats."""
    if visible < 1:
        raise ValueError("at least one key must be visible")
    scores = []
    for j in range(visible):
        acc = 0.0
        for a, b in zip(q, keys[j]):
            acc += a * b
        scores.append(scale * acc)
    m = max(scores)
    weights = [math.exp(s - m) for s in scores]
    z = math.fsum(weights)
    dim = len(values[0])
    out = []
    for d in range(dim):
        out.append(math.fsum(weights[j] * values[j][d] for j in range(visible)) / z)
    return out
