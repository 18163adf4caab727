"""Pure-Python attention on logical (contiguous) K/V lists, for tiny inputs.

No numpy, no paging: triple loops over scores, a max-shifted exponential and a
weighted sum, in Python floats (fp64).  It is the textbook softmax(q K^T s) V
and knows nothing of blocks, tables or tile layouts.
"""
import math


def attend(q, keys, values, scale):
    """q: [D]; keys, values: [n][D] lists of floats.  Returns [D]."""
    n = len(keys)
    D = len(q)
    if n == 0:
        return [0.0] * D
    scores = []
    for t in range(n):
        acc = 0.0
        for d in range(D):
            acc += q[d] * keys[t][d]
        scores.append(acc * scale)
    m = max(scores)
    weights = [math.exp(z - m) for z in scores]
    total = sum(weights)
    out = []
    for d in range(D):
        acc = 0.0
        for t in range(n):
            acc += weights[t] * values[t][d]
        out.append(acc / total)
    return out
