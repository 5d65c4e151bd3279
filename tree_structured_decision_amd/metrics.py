"""Host-side evaluation of layer outputs: per-option scores, total-variation
distance and decision agreement.

Fidelity is measured by the total-variation distance (half the L1 distance) of
output probabilities to a float32 reference (Flide, kongchang.com page,
section "Performance"), and by whether accelerated runs keep the same
decisions (openai-hub.com page, section on accuracy and calibration).

Reading used here (the pages define no readout): a decision group is the set
of leaf segments sharing one parent; option c's score is
<w, vec(o at c's last token)> / sqrt(len(w)) with a seeded readout vector w,
and the group's probabilities are the float64 softmax of its scores.
"""
from __future__ import annotations

import numpy as np

from .workloads import group_options


def option_scores(o: np.ndarray, w: np.ndarray, parent, seg_len) -> dict:
    """{parent: (leaf segments, scores)} for every decision group."""
    o = np.asarray(o, np.float64)
    seg_len = np.asarray(seg_len, np.int64)
    start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    w = np.asarray(w, np.float64)
    out = {}
    for p, leaves in group_options(parent, seg_len):
        rows = np.stack([o[start[c] + seg_len[c] - 1].reshape(-1) for c in leaves])
        out[p] = (leaves, rows @ w / np.sqrt(w.size))
    return out


def softmax64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def tvd(p: np.ndarray, q: np.ndarray) -> float:
    return 0.5 * float(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum())


def decision_fidelity(o_test: np.ndarray, o_ref: np.ndarray, w: np.ndarray, parent, seg_len) -> dict:
    """Max / mean TVD over decision groups and argmax agreement rate (ties go
    to the lowest index, as np.argmax does)."""
    st = option_scores(o_test, w, parent, seg_len)
    sr = option_scores(o_ref, w, parent, seg_len)
    tv, agree = [], []
    for p in sr:
        pt, pr = softmax64(st[p][1]), softmax64(sr[p][1])
        tv.append(tvd(pt, pr))
        agree.append(int(np.argmax(pt) == np.argmax(pr)))
    if not tv:
        return dict(groups=0, tvd_max=0.0, tvd_mean=0.0, argmax_agreement=1.0)
    return dict(groups=len(tv), tvd_max=float(np.max(tv)), tvd_mean=float(np.mean(tv)),
                argmax_agreement=float(np.mean(agree)))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (0 for x == 0)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)
