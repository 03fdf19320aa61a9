"""Per-token log-probability difference of two policies, in fp64.

Test infrastructure only (see the package header).

[P2] "Five design features of the adapter-first architecture": the KL
regulariser of RL post-training compares the trained policy (base + OFT
adapter) with a reference policy, and the reference is the frozen base run
without the adapter, so no second model is kept.  The KL term is estimated
from the log-probabilities the two policies give the sampled token:
    d[t] = log softmax(a[t])[label[t]] - log softmax(r[t])[label[t]],
with a, r the two policies' logits over the vocabulary.  This is that
definition written out: log softmax(v)[i] = v[i] - log(sum_j exp(v[j])),
the sum taken after subtracting the row maximum.
"""
from __future__ import annotations

import numpy as np


def log_softmax_at(logits: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """log softmax of every row of logits [T, V] at labels [T], fp64."""
    L = np.asarray(logits, dtype=np.float64)
    mx = L.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(L - mx).sum(axis=1))
    return L[np.arange(L.shape[0]), np.asarray(labels, dtype=np.int64)] - lse


def logprob_diff(actor: np.ndarray, ref: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """d[t] = log p_actor(label[t] | t) - log p_ref(label[t] | t)."""
    return log_softmax_at(actor, labels) - log_softmax_at(ref, labels)
