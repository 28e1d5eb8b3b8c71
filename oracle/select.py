"""Row argmax and the sharpened draft child selection.

TEST INFRASTRUCTURE ONLY (see the package header).

Greedy verification takes the target's argmax at each tree node ([Review] §3.2,
temperature 0). SubSpec sharpens the draft distribution with temperature 0.2
([Summary] "Approach" and "Measured effects reported in the paper"; [Review] §3.4)
and keeps k = 6 children per node ([Review] §6.3). The pages do not say how the
children are drawn. Reading: Gumbel-top-k, i.e. sampling k tokens without
replacement from softmax(logits / t): add independent Gumbel(0,1) noise g to
logits / t and keep the k largest. g = 0 gives plain top-k (greedy drafting).

Bit-exact rules: y = fp32(fp32(logit * inv_t) + g), two fp32 operations rounded to
nearest-even, no FMA; order by y descending, equal y by lower token index first;
argmax takes the lowest index among equal maxima.
"""

import numpy as np


def row_argmax(logits) -> np.ndarray:
    return np.argmax(np.asarray(logits, dtype=np.float32), axis=1).astype(np.int32)


def draft_select(logits, gumbel, inv_temp, k) -> np.ndarray:
    """Top-k token indices per row of y = logits * inv_temp (+ gumbel), int32 [R][k]."""
    lg = np.asarray(logits, dtype=np.float32)
    y = lg * np.float32(inv_temp)
    if gumbel is not None:
        y = y + np.asarray(gumbel, dtype=np.float32)
    R, V = y.shape
    idx = np.arange(V)
    out = np.empty((R, k), dtype=np.int32)
    for r in range(R):
        order = np.lexsort((idx, -y[r]))
        out[r] = order[:k]
    return out
