"""fp64 model of the tiled online-softmax recurrence -- TEST INFRASTRUCTURE ONLY.

This follows the "FLASH" half of the naive-vs-flash diagram on the mlapandio
page "FlashAttention: IO-aware exact attention". For each block of query rows,
the running output O, max m and sum l start at 0, -inf and 0. Each streamed
key/value block then updates them:

    m_new = max(m, rowmax(S_tile))
    l     = e^(m - m_new) * l + rowsum(e^(S_tile - m_new))
    O     = e^(m - m_new) * O + e^(S_tile - m_new) V_block
    m     = m_new

The diagram ends by storing the accumulated O and one logsumexp per row, and
leaves the final normalisation open. The reading used here is the only one
under which the running statistics reproduce the ordinary softmax, as the
page's "Four ideas" section says they do: O is divided by l, and
LSE = m + ln l.

``tau`` models a lazily updated reference max. The reference m moves only when
a block's row max exceeds it by more than ``tau`` (natural-log units).

``sum_max`` models the rule the HIP forward kernel uses instead. The reference
starts at the first key block's row max. For each later block the
probabilities e^(S - m) are formed under the old reference; only when some row
of the row block sums past ``sum_max`` (or overflows) does the whole row block
move to m = max(m, rowmax). No row max is needed for the other blocks.

Any reference value cancels in O / l and in m + ln l, so the result is the
same under every rule; the tests check that in fp64.

The model is numpy fp64 with a numpy matmul as its product step. It serves
only to pin the algorithm's order of steps against the definition.
"""
from __future__ import annotations

import numpy as np


def online_attention(q, k, v, causal: bool, scale: float, block_rows: int, block_cols: int,
                     tau: float = 0.0, sum_max: float | None = None):
    """q [Nq, d], k/v [Nk, d] float64 for one head (queries at positions 0..Nq-1).
    Returns O [Nq, d], LSE [Nq]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, d = q.shape
    Nk = k.shape[0]
    O_out = np.zeros((Nq, d))
    L_out = np.zeros(Nq)
    for r0 in range(0, Nq, block_rows):
        rows = np.arange(r0, min(r0 + block_rows, Nq))
        Qb = q[rows]
        O = np.zeros((len(rows), d))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        for c0 in range(0, Nk, block_cols):
            cols = np.arange(c0, min(c0 + block_cols, Nk))
            S = scale * (Qb @ k[cols].T)
            if causal:
                S = np.where(cols[None, :] <= rows[:, None], S, -np.inf)
            rowmax = S.max(axis=1)
            if sum_max is None:
                # lazy reference: move m only when the block max clears it by more than tau
                move = (rowmax > m + tau) | np.isneginf(m)
            else:
                # move the whole row block when some row's probabilities under the
                # old reference sum past sum_max (the first block always moves)
                with np.errstate(over="ignore", invalid="ignore"):
                    sums = np.exp(S - m[:, None]).sum(axis=1)
                grow = bool(np.any(~(sums <= sum_max))) or bool(np.any(np.isneginf(m)))
                move = np.full(len(rows), grow)
            m_new = np.where(move, np.maximum(m, rowmax), m)
            # a row with no visible key so far keeps m = -inf; its terms are all zero
            safe = np.where(np.isneginf(m_new), 0.0, m_new)
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - safe))
            E = np.exp(S - safe[:, None])
            l = alpha * l + E.sum(axis=1)
            O = alpha[:, None] * O + E @ v[cols]
            m = m_new
        O_out[rows] = O / l[:, None]
        L_out[rows] = m + np.log(l)
    return O_out, L_out
