"""Oracle of the per-option decision readout.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
smoke check and the benchmark's CPU-baseline leg are its only callers.

The pages measure a decision engine by the probabilities it gives each
candidate option: their distance to a float32 reference in total variation
(kongchang.com page, section on performance) and whether the chosen option
stays the same (openai-hub.com page, section on the six variables). They do
not define the readout itself. Reading taken: a decision group is the set of
leaf segments (options) that share one parent segment; option c's score is

    score[c] = <w, x[last token of c]> / sqrt(len(w))

with x a layer's output rows flattened per token ([T, C]) and w a readout
vector of C values; the group's probabilities are the softmax of its
scores. Every other segment (interior segments, roots without children) is
not an option: its score and probability are 0.

Plain float64 numpy, one loop over segments, one over groups.
"""
from __future__ import annotations

import numpy as np


def option_readout(x: np.ndarray, w: np.ndarray, parent, seg_len):
    """(score[S], prob[S]) in float64, following the definition above."""
    parent = np.asarray(parent, np.int64)
    seg_len = np.asarray(seg_len, np.int64)
    S = parent.shape[0]
    x = np.asarray(x, np.float64).reshape(int(seg_len.sum()), -1)
    w = np.asarray(w, np.float64).reshape(-1)
    if x.shape[1] != w.size:
        raise ValueError(f"rows of {x.shape[1]} values, readout vector of {w.size}")
    start = np.zeros(S, np.int64)
    for s in range(1, S):
        start[s] = start[s - 1] + seg_len[s - 1]
    has_child = np.zeros(S, bool)
    for s in range(S):
        if parent[s] >= 0:
            has_child[parent[s]] = True
    is_option = np.array([parent[s] >= 0 and not has_child[s] for s in range(S)])

    score = np.zeros(S, np.float64)
    for s in range(S):
        if is_option[s]:
            last = x[start[s] + seg_len[s] - 1]
            score[s] = float(np.dot(w, last)) / np.sqrt(w.size)

    prob = np.zeros(S, np.float64)
    for p in range(S):
        members = [s for s in range(S) if is_option[s] and parent[s] == p]
        if not members:
            continue
        z = score[members]
        e = np.exp(z - z.max())
        prob[members] = e / e.sum()
    return score, prob
