"""GPU decision readout (fork_option_readout) against the readout oracle
(oracle/readout.py), through the C ABI, on the same input rows.

Both sides read the same values (bf16 inputs are decoded exactly into the
oracle's float64). The bars follow from the kernel's fp32 arithmetic, with
u = 2^-24:
- score: each lane sums C/64 products in order, a 6-level butterfly adds the
  64 partials, and one product applies 1/sqrt(C) (rounded once, applied with
  one more rounding), so |score - ref| <= (C/64 + 10) u sum_i |w_i x_i| / sqrt(C);
- probability: scores off by at most e move a group's probabilities by a
  factor within exp(+-2e); expf (1 ulp), the running rescales and the n-term
  sum of a group of n options, and the final product add at most (n + 16)
  units of 2^-23 relative, so |p - ref| <= ref (exp(2e) - 1 + (n + 16) 2^-23).
Segments that are not options must read exactly 0. Cases: hand-built forests
with nested groups, non-contiguous siblings and ragged rows, bf16 and fp32,
C from 8 to 4096; the request mix at full size (2,891 segments, groups of 2
to 256 options, 316,934 rows of 2,048 values); repeated calls bit for bit."""
import zlib

import numpy as np
import pytest
import torch

from oracle.readout import option_readout
from tests.gpu_helpers import log
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _bars(x_last, w, parent, score_ref, prob_ref):
    """Per-segment score and probability bars (see the module docstring)."""
    C = w.size
    mag = np.abs(x_last * w[None, :]).sum(axis=1) / np.sqrt(C)
    e_score = (C / 64 + 10) * U * mag
    S = len(parent)
    has_child = np.zeros(S, bool)
    has_child[parent[parent >= 0]] = True
    option = (parent >= 0) & ~has_child
    e_prob = np.zeros(S)
    for p in np.unique(parent[option]):
        members = np.where(option & (parent == p))[0]
        e = e_score[members].max()
        e_prob[members] = prob_ref[members] * (np.expm1(2 * e) + (len(members) + 16) * 2.0 ** -23)
    return e_score, e_prob, option


def _check(name, parent, seg_len, x_dev, x_last, w, sess):
    w_dev = torch.from_numpy(w.astype(np.float32)).cuda()
    w64 = w.astype(np.float32).astype(np.float64)
    score, prob = sess.option_readout(x_dev, w_dev)
    score2, prob2 = sess.option_readout(x_dev, w_dev)
    torch.cuda.synchronize()
    s_gpu, p_gpu = score.cpu().numpy().astype(np.float64), prob.cpu().numpy().astype(np.float64)
    assert torch.equal(score, score2) and torch.equal(prob, prob2), f"{name}: repeated calls differ"
    ones = np.ones(len(parent), np.int64)
    s_ref, p_ref = option_readout(x_last, w64, parent, ones)  # only each segment's last row is read
    e_s, e_p, option = _bars(x_last, w64, np.asarray(parent), s_ref, p_ref)
    assert np.all(s_gpu[~option] == 0.0) and np.all(p_gpu[~option] == 0.0), f"{name}: non-options not zero"
    ds, dp = np.abs(s_gpu - s_ref), np.abs(p_gpu - p_ref)
    log(f"{name}: {option.sum()} options, max |score err| {ds.max():.3g} (bar {e_s[option].max():.3g}), "
        f"max |prob err| {dp.max():.3g} (bar {e_p[option].max():.3g})")
    assert np.all(ds <= e_s + 1e-30), f"{name}: score error {ds.max()} above its bar"
    assert np.all(dp <= e_p + 1e-30), f"{name}: probability error {dp.max()} above its bar"


FORESTS = {
    # root with interior child 1 (leaves 4, 5) and leaves 2, 3; siblings 2, 3 interleave with 4
    "nested": ([-1, 0, 0, 1, 0, 1, 3, 3], [5, 3, 1, 2, 4, 7, 1, 2]),
    # two roots, one without children, a chain whose only leaf is deep
    "roots_chain": ([-1, -1, 1, 2, 3, 1, 1], [3, 2, 4, 1, 6, 2, 2]),
    # one group of 40 options of ragged lengths
    "wide": ([-1] + [0] * 40, [17] + [1 + (i * 7) % 11 for i in range(40)]),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [8, 520, 4096])
@pytest.mark.parametrize("forest", list(FORESTS))
def test_readout_small(forest, C, dtype):
    parent = np.array(FORESTS[forest][0], np.int32)
    seg_len = np.array(FORESTS[forest][1], np.int32)
    rng = np.random.default_rng(zlib.crc32(f"{forest}/{C}/{dtype}".encode()))
    T = int(seg_len.sum())
    x = rng.standard_normal((T, C)).astype(np.float32) * 2.0
    w = rng.standard_normal(C).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x_dev = torch.from_numpy(x).cuda().to(tdt)
    x64 = x_dev.float().cpu().numpy().astype(np.float64)
    last = np.cumsum(seg_len) - 1
    caps = caps_for(parent, seg_len, 1)
    sess = ForkSession(**caps, D=64, gH=1, dk=64, dv=64, device="cuda")
    try:
        sess.build(parent, seg_len)
        _check(f"{forest} C={C} {dtype}", parent, seg_len, x_dev, x64[last], w, sess)
    finally:
        sess.close()


def test_readout_request_mix_full_size():
    """The request mix's tree (seed of the bench): rows of 16 x 128 bf16 values.
    Every row that is not a segment's last holds 1000 (a read of a wrong row
    would show); each last row holds seeded N(0, 1) values."""
    rng = np.random.default_rng(2024)
    parent, seg_len = W.request_mix_tree(np.random.Generator(np.random.PCG64(W.SEED_BASE + 5)), 64)
    parent = np.asarray(parent, np.int32)
    seg_len = np.asarray(seg_len, np.int32)
    T, S, C = int(seg_len.sum()), len(parent), 16 * 128
    log(f"request mix readout: T={T} S={S} C={C}")
    last = np.cumsum(seg_len.astype(np.int64)) - 1
    x_last = rng.standard_normal((S, C)).astype(np.float32)
    x_dev = torch.full((T, C), 1000.0, dtype=torch.bfloat16, device="cuda")
    rows = torch.from_numpy(x_last).cuda().to(torch.bfloat16)
    x_dev.index_copy_(0, torch.from_numpy(last).cuda(), rows)
    x64 = rows.float().cpu().numpy().astype(np.float64)
    w = rng.standard_normal(C).astype(np.float32)
    caps = caps_for(parent, seg_len, 8)
    sess = ForkSession(**caps, D=128, gH=16, dk=128, dv=128, device="cuda")
    try:
        sess.build(parent, seg_len)
        _check("request mix", parent, seg_len, x_dev, x64, w, sess)
    finally:
        sess.close()


def test_readout_graph_replay_matches_eager():
    """fork_option_readout recorded once in a graph (for one tree) and replayed
    four times on two trees built in turn into the same blob, with the inputs
    rewritten and the outputs poisoned between replays: every replay equals
    the eager call on that tree bit for bit, and the eager calls meet the
    oracle bars."""
    C = 520
    trees = [FORESTS["nested"], FORESTS["wide"]]
    trees = [(np.array(p, np.int32), np.array(l, np.int32)) for p, l in trees]
    t_cap = max(int(l.sum()) for _, l in trees)
    s_cap = max(len(p) for p, _ in trees)
    depth = max(caps_for(p, l, 1)["depth_cap"] for p, l in trees)
    sess = ForkSession(t_cap=t_cap, s_cap=s_cap, depth_cap=depth, gqa_group=1, D=64, gH=1, dk=64, dv=64,
                       device="cuda")
    rng = np.random.default_rng(99)
    xs = [rng.standard_normal((t_cap, C)).astype(np.float32) for _ in trees]
    x = torch.empty((t_cap, C), dtype=torch.bfloat16, device="cuda")
    w = torch.from_numpy(rng.standard_normal(C).astype(np.float32)).cuda()
    score = torch.empty(s_cap, dtype=torch.float32, device="cuda")
    prob = torch.empty(s_cap, dtype=torch.float32, device="cuda")
    try:
        def load(i):
            sess.build(*trees[i])
            x.copy_(torch.from_numpy(xs[i]).to(torch.bfloat16))

        eager = []
        for i, (parent, seg_len) in enumerate(trees):
            load(i)
            sess.option_readout(x, w, score, prob)
            torch.cuda.synchronize()
            S = len(parent)
            eager.append((score[:S].clone(), prob[:S].clone()))
            x64 = x.float().cpu().numpy().astype(np.float64)
            _check(f"graph tree {i}", parent, seg_len, x, x64[np.cumsum(seg_len) - 1], w.cpu().numpy(), sess)
        load(0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sess.option_readout(x, w, score, prob)
        for rep, i in enumerate((0, 1, 0, 1)):
            load(i)
            score.fill_(float("nan"))
            prob.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            S = len(trees[i][0])
            assert torch.equal(score[:S], eager[i][0]) and torch.equal(prob[:S], eager[i][1]), f"replay {rep}"
            log(f"  readout replay {rep} (tree {i}) equals the eager call")
        del graph
    finally:
        sess.close()
