"""Plain softmax attention and the softmax variational objective, in float64.

Test infrastructure only (see the package docstring).

The variational form of softmax ([MA] scime summary "Proposal"/"Approach";
OpenReview author response on convergence, which calls it equation (6), and on
concavity): for a score row s, softmax(s) is the maximiser over the probability
simplex of  <p, s> + H(p),  with H(p) = -sum p log p, and the maximum equals
logsumexp(s).  For an attention matrix M with simplex rows and scores S,

    f(M) = sum_rows ( <M_row, S_row> + H(M_row) ),

maximised by row-wise softmax(S) with value sum_rows logsumexp(S_row).

Pins: exact_attention is checked against torch's CPU scaled-dot-product
attention and against a hand-expanded 2x2 case; dense_objective against the
closed form f(softmax(S)) = sum logsumexp(S) and f(M) = sum lse - sum KL.
"""

import numpy as np


def logsumexp(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def softmax(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def row_entropy(p, axis=-1):
    """H(p) = -sum p log p, with 0 log 0 = 0."""
    safe = np.where(p > 0, p, 1.0)
    return -np.sum(np.where(p > 0, p * np.log(safe), 0.0), axis=axis)


def exact_attention(q, k, v, scale):
    """Y = softmax(scale * Q K^T) V for one (batch, head) slice; q,k,v [N, d]."""
    s = scale * (q @ k.T)
    return softmax(s, axis=-1) @ v


def dense_objective(m, s):
    """f(M) = sum over rows of <M_row, S_row> + H(M_row)  (M, S: [N, N])."""
    return float(np.sum(m * s) + np.sum(row_entropy(m, axis=-1)))
