"""N-gram prompt-lookup drafter for the synthetic verify step.

The pages compare Quasar against an N-gram drafter verified in BF16 [Quasar,
ko page §4 results table; zh page §4]: drafts are copied from earlier text
that continues the most recent n tokens.  The pages give no parameters, so:

* the longest n-gram first, from ``n_max`` down to 1;
* the most recent earlier occurrence of the history's last n tokens wins;
* the draft is the k tokens that followed that occurrence; a continuation
  shorter than k is padded with its own last token, and with no match at any
  n the draft is k copies of the last token.

Host-side logic on token ids (numpy); it runs between verify steps, not on
the GPU.
"""
from __future__ import annotations

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view


def ngram_draft(history: np.ndarray, k: int, n_max: int = 3) -> np.ndarray:
    """k draft tokens (int32) continuing ``history`` (1-D token ids, length >= 1)."""
    h = np.asarray(history, dtype=np.int64)
    n = len(h)
    if n == 0:
        raise ValueError("history must hold at least one token")
    if k <= 0:
        return np.zeros(0, np.int32)
    for g in range(min(n_max, n - 1), 0, -1):
        suffix = h[n - g:]
        windows = sliding_window_view(h[:n - 1], g)  # starts 0 .. n - 1 - g
        hits = np.flatnonzero(np.all(windows == suffix[None, :], axis=1))
        hits = hits[hits < n - g]  # an earlier occurrence, not the suffix itself
        if len(hits):
            p = int(hits[-1])
            cont = h[p + g:p + g + k]
            if len(cont):
                out = np.full(k, cont[-1], np.int64)
                out[:len(cont)] = cont
                return out.astype(np.int32)
    return np.full(k, h[-1], np.int32)
