"""Per-iteration residual-norm safety check, plain float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Current Status" page, architecture-unique features table: after every loop
iteration the L2 norm of the residual stream is computed and the forward is
aborted when it exceeds a threshold (L checkpoints per token). Reading taken
where the page is silent: the check runs on every row (token) of the call
after each loop iteration i = 0..L-1 (pre-blocks are not checked); the first
trip in (iteration, row) order is reported; a NaN norm trips too.
"""
from __future__ import annotations

import numpy as np

from .model import forward


def safety_trip(model, tokens, L, max_norm, cache=None, max_seq=None, kv_int8=False, window=0):
    """First (iteration, row, norm) whose residual L2 norm is not <= max_norm,
    or None, for a forward of `tokens` at depth L (appended to `cache`)."""
    s = model.shape
    r = forward(model, tokens, L, cache=cache, logits=None, trace=True, max_seq=max_seq,
                kv_int8=kv_int8, window=window)
    for i in range(L):
        x = r["trace"][s.n_pre + i]
        norms = np.sqrt((x * x).sum(axis=1))
        bad = np.nonzero(~(norms <= max_norm))[0]
        if bad.size:
            return i, int(bad[0]), float(norms[bad[0]])
    return None
