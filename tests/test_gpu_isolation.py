"""The method's guarantee end to end on the GPU (kongchang.com page, section
"ForkAttention: exact forking in GPU indices": each branch evaluates as its
isolated forward pass): a four-layer hybrid stack run once over a forest
gives, for every leaf, the rows that the same stack gives when that leaf's
root-to-leaf path is run alone as one sequence, in bf16 and with FP8
projections (per-token activation scales keep each token's codes independent
of the other branches).

Bar: the two GPU runs differ only in accumulation order (other tilings, key
splits and product algorithms for the other stream length), so the rows
agree within relative RMS 1e-2 (bf16) / 3e-2 (FP8), the bars of the stack
parity tests, and every decision group's option softmax within TVD 1e-2."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import log
from tests.test_gpu_mixer import dev, dev_stack, host, session
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd import workloads as W

pytestmark = pytest.mark.gpu


def path_rows(parent, seg_len, leaf):
    start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    segs = []
    s = leaf
    while s >= 0:
        segs.append(s)
        s = parent[s]
    return np.concatenate([np.arange(start[s], start[s] + seg_len[s]) for s in segs[::-1]])


@pytest.mark.parametrize("fp8", [False, True])
def test_stack_branches_equal_isolated_runs(fp8):
    rng = np.random.default_rng(131)
    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 2, 3, 3], np.int32)
    seg_len = rng.integers(1, 60, parent.size).astype(np.int32)
    seg_len[0] = 150
    seg_len[[4, 7]] = 1
    T = int(seg_len.sum())
    heads = dict(H=4, Hkv=2, D=64, gH=2, dk=64, dv=64)
    layers, fn, w_head = W.stack_weights(132, 256, **heads)
    x = W.mixer_input(133, T, 256)

    def run(par, lens, xs):
        sess = session(par, lens, group=2, kv_heads=2, D=64, gH=2, dk=64, dv=64)
        dl, dfn = dev_stack(layers, fn, "bf16")
        if fp8:
            dl = [(k, sess.quantize_weights(Wl), nw) for k, Wl, nw in dl]
        h = host(sess.stack(dev(xs, "bf16"), dl, dfn, fp8=fp8))
        sess.close()
        return h

    h_tree = run(parent, seg_len, x)
    leaves = [s for s in range(parent.size) if not (parent == s).any()]
    iso = np.full_like(h_tree, np.nan)
    worst = 0.0
    for leaf in leaves:
        rows = path_rows(parent, seg_len, leaf)
        h_path = run(np.array([-1], np.int32), np.array([rows.size], np.int32), x[rows])
        rel = np.linalg.norm(h_path - h_tree[rows]) / np.linalg.norm(h_tree[rows])
        worst = max(worst, rel)
        assert rel <= (3e-2 if fp8 else 1e-2), (leaf, rel)
        last = rows[-1]
        iso[last] = h_path[-1]
    fid = metrics.decision_fidelity(np.where(np.isnan(iso), h_tree, iso), h_tree, w_head, parent, seg_len)
    log(f"  {'fp8' if fp8 else 'bf16'} stack, {len(leaves)} leaves: worst path relative RMS {worst:.2e}, "
        f"option softmax isolated vs tree: {fid}")
    assert fid["groups"] == 3 and fid["tvd_max"] <= 1e-2
