"""Pins of the decision-readout oracle (oracle/readout.py).

The readout is a reading (the pages define no scoring head): options are the
leaf segments, grouped by their parent; score = <w, last row> / sqrt(C);
probabilities = softmax within the group. The pins below fix it without
re-typing its formula:

- a hand-worked tree whose expected values are derived on paper. It is built
  so that a readout of the first token instead of the last (segment 5 has two
  tokens that differ), grouping by root instead of by parent (it would merge
  groups {2, 3} and {4, 5}), treating interior segments as options (segment 1
  has children), or dropping the 1/sqrt(C) factor each changes a value;
- the group probabilities equal scipy's softmax of the group's scores;
- a shift of every option's last row along w shifts all scores by the same
  amount and leaves the probabilities unchanged;
- swapping two sibling options in the stream swaps their outputs.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special

from oracle.readout import option_readout


def _hand_tree():
    # segment: 0 root (2 tokens), 1 child of 0 with two leaf children (4, 5),
    # 2 and 3 leaf children of 0; 5 has two tokens.
    parent = [-1, 0, 0, 0, 1, 1]
    seg_len = [2, 1, 1, 1, 1, 2]
    T, C = sum(seg_len), 4
    x = np.full((T, C), 7.0)          # every row not named below: 7 in the read coordinate
    x[:, 1:] = [1.0, -2.0, 5.0]       # coordinates that w ignores
    # token index of each segment's rows: 0:[0,1] 1:[2] 2:[3] 3:[4] 4:[5] 5:[6,7]
    x[3, 0] = 0.0                     # last (only) row of option 2
    x[4, 0] = 2.0 * math.log(3.0)     # option 3
    x[5, 0] = 2.0                     # option 4
    x[6, 0] = -40.0                   # first row of option 5 (must not be read)
    x[7, 0] = 2.0                     # last row of option 5
    w = np.array([1.0, 0.0, 0.0, 0.0])
    return parent, seg_len, x, w


def test_hand_worked_tree():
    parent, seg_len, x, w = _hand_tree()
    score, prob = option_readout(x, w, parent, seg_len)
    # score = x[last, 0] * 1 / sqrt(4)
    np.testing.assert_allclose(score, [0.0, 0.0, 0.0, math.log(3.0), 1.0, 1.0], rtol=0, atol=1e-15)
    # group {2, 3}: e^0 : e^{ln 3} = 1 : 3; group {4, 5}: equal scores
    np.testing.assert_allclose(prob, [0.0, 0.0, 0.25, 0.75, 0.5, 0.5], rtol=0, atol=1e-15)


def _random_forest(rng, n_roots=3):
    parent, seg_len = [], []
    for _ in range(n_roots):
        r = len(parent)
        parent.append(-1)
        seg_len.append(int(rng.integers(1, 9)))
        kids = []
        for _ in range(int(rng.integers(0, 4))):
            kids.append(len(parent))
            parent.append(r)
            seg_len.append(int(rng.integers(1, 6)))
        for kid in kids[:1]:
            for _ in range(int(rng.integers(1, 5))):
                parent.append(kid)
                seg_len.append(int(rng.integers(1, 6)))
    return np.array(parent), np.array(seg_len)


@pytest.mark.parametrize("seed", range(6))
def test_probabilities_are_scipy_softmax_of_group_scores(seed):
    rng = np.random.default_rng(seed)
    parent, seg_len = _random_forest(rng)
    C = 16
    x = rng.standard_normal((int(seg_len.sum()), C)) * 3.0
    w = rng.standard_normal(C)
    score, prob = option_readout(x, w, parent, seg_len)
    S = len(parent)
    has_child = np.zeros(S, bool)
    has_child[parent[parent >= 0]] = True
    options = [s for s in range(S) if parent[s] >= 0 and not has_child[s]]
    for s in range(S):
        if s not in options:
            assert score[s] == 0.0 and prob[s] == 0.0
    for p in set(int(parent[s]) for s in options):
        members = [s for s in options if parent[s] == p]
        np.testing.assert_allclose(prob[members], scipy.special.softmax(score[members]), rtol=1e-13, atol=0)
        assert abs(prob[members].sum() - 1.0) < 1e-13


def test_shift_along_w_moves_scores_not_probabilities():
    rng = np.random.default_rng(11)
    parent, seg_len = _random_forest(rng, n_roots=4)
    C = 8
    x = rng.standard_normal((int(seg_len.sum()), C))
    w = rng.standard_normal(C)
    s0, p0 = option_readout(x, w, parent, seg_len)
    delta = 0.75
    x1 = x + delta * math.sqrt(C) * w / np.dot(w, w)   # every row: <w, row> grows by delta sqrt(C)
    s1, p1 = option_readout(x1, w, parent, seg_len)
    opt = p0 > 0
    np.testing.assert_allclose(s1[opt] - s0[opt], delta, rtol=0, atol=1e-12)
    np.testing.assert_allclose(p1, p0, rtol=0, atol=1e-14)


def test_swapping_sibling_options_swaps_outputs():
    # root (3 tokens) with three leaf options of lengths 2, 4, 3; swap options 1 and 3.
    rng = np.random.default_rng(5)
    C = 8
    rows = {0: rng.standard_normal((3, C)), 1: rng.standard_normal((2, C)),
            2: rng.standard_normal((4, C)), 3: rng.standard_normal((3, C))}
    w = rng.standard_normal(C)
    order_a, order_b = [0, 1, 2, 3], [0, 3, 2, 1]
    xa = np.concatenate([rows[s] for s in order_a])
    xb = np.concatenate([rows[s] for s in order_b])
    sa, pa = option_readout(xa, w, [-1, 0, 0, 0], [rows[s].shape[0] for s in order_a])
    sb, pb = option_readout(xb, w, [-1, 0, 0, 0], [rows[s].shape[0] for s in order_b])
    np.testing.assert_array_equal(sb[[0, 3, 2, 1]], sa)
    np.testing.assert_allclose(pb[[0, 3, 2, 1]], pa, rtol=1e-15, atol=0)  # the group sum runs in another order
