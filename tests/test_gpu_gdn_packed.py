"""Gated DeltaNet without end states: the scan packs runs of consecutive leaf
siblings (at most one 64-token chunk in total) into one chunk that starts
from their parent's state, with the decays restarting at each sibling and the
intra-chunk products masked to same-sibling pairs. Checked against the oracle
(outputs and start states) on trees built level by level, so that siblings
are consecutive: many short leaves, leaves longer than a chunk, runs of
siblings that overflow a chunk, inner children with their own children, and
several roots with given root states; on the three-level agent history at
full size (sampled segments); and bit for bit against the same launch with
end states requested, whose start states (every fork copy comes from a
parent that is never packed) must not change."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import check_close, log, oracle_gdn
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

pytestmark = pytest.mark.gpu


def level_tree(rng, roots=2, depth=3, kids=(2, 12), inner=0.3):
    """Parents before children, each parent's children consecutive. Lengths:
    mostly short leaves (1-40 tokens), some longer than a chunk."""
    parent, seg_len = [], []

    def length():
        u = rng.random()
        return int(rng.integers(1, 9)) if u < 0.4 else int(rng.integers(9, 41)) if u < 0.85 else int(
            rng.integers(65, 160))

    level = []
    for _ in range(roots):
        parent.append(-1)
        seg_len.append(int(rng.integers(70, 300)))
        level.append(len(parent) - 1)
    for d in range(1, depth):
        nxt = []
        for p in level:
            for _ in range(int(rng.integers(kids[0], kids[1] + 1))):
                parent.append(p)
                seg_len.append(length())
                if d + 1 < depth and rng.random() < inner:
                    nxt.append(len(parent) - 1)
        level = nxt
    return np.array(parent, np.int32), np.array(seg_len, np.int32)


def run_gdn(wl, final):
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv)
    sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
    d = to_device(wl, "cuda")
    sess.build(wl.parent, wl.seg_len)
    go = torch.full((wl.T, wl.gH, wl.dv), float("nan"), device="cuda", dtype=d["gq"].dtype)
    st0 = torch.full((wl.S, wl.gH, wl.dv, wl.dk), float("nan"), device="cuda")
    st1 = torch.full_like(st0, float("nan")) if final else None
    sess.gdn(d["gq"], d["gk"], d["gv"], d["a"], d["b"], go, st0, st1, root_state=d["root_state"])
    torch.cuda.synchronize()
    assert sess.check() == 0
    out = {"go": go, "s0": st0}
    if final:
        out["s1"] = st1
    res = {k: v.float().cpu().numpy() for k, v in out.items()}
    sess.close()
    return res


def packed_runs(parent, seg_len):
    """Number of leaf-sibling runs the plan packs (for the log)."""
    S = len(parent)
    has_kid = np.zeros(S, bool)
    has_kid[parent[parent >= 0]] = True
    leaf = (parent >= 0) & ~has_kid & (seg_len <= 64)
    n, tot = 0, 0
    for s in range(S):
        if leaf[s] and s > 0 and leaf[s - 1] and parent[s] == parent[s - 1] and tot + seg_len[s] <= 64:
            tot += seg_len[s]
            continue
        n += int(leaf[s])
        tot = seg_len[s] if leaf[s] else 0
    return n, int(leaf.sum())


@pytest.mark.parametrize("seed,gates,roots", [(11, "uniform", 1), (12, "sigmoid", 3), (13, "uniform", 2)])
def test_packed_leaves_match_oracle(seed, gates, roots):
    rng = np.random.default_rng(seed)
    parent, seg_len = level_tree(rng, roots=roots)
    wl = W.make_workload("packed", "bf16", parent, seg_len, H=4, Hkv=2, D=64, gH=2, dk=128, dv=128,
                         gates=gates, root_state_std=0.5 if roots > 1 else None, seed=seed)
    n_runs, n_leaves = packed_runs(parent, seg_len)
    log(f"tree: S={wl.S} T={wl.T}; {n_leaves} short leaves in {n_runs} packed chunks")
    got = run_gdn(wl, final=False)
    go, s0, _ = oracle_gdn(wl)
    check_close("gdn.o (packed)", got["go"], go, "bf16")
    check_close("gdn.start_state (packed)", got["s0"], s0, "bf16", kind="f32")
    ref = run_gdn(wl, final=True)
    np.testing.assert_array_equal(got["s0"].view(np.int32), ref["s0"].view(np.int32))
    check_close("gdn.o (packed vs unpacked)", got["go"], ref["go"], "bf16")


def test_packed_agent_history_sampled():
    wl = W.agent_history()
    got = run_gdn(wl, final=False)
    segs = [0, 3, 9, 100, 264, wl.S - 1]
    sel = np.zeros(wl.S, np.uint8)
    sel[segs] = 1
    go, s0, _ = oracle_gdn(wl, seg_select=sel)
    st = np.concatenate([[0], np.cumsum(wl.seg_len)[:-1]])
    rows = np.zeros(wl.T, bool)
    for s in segs:
        rows[st[s]:st[s] + wl.seg_len[s]] = True
    check_close("gdn.o[sampled] (packed)", got["go"], go, wl.dtype, rows=rows)
    check_close("gdn.start_state[sampled] (packed)", got["s0"], s0, wl.dtype, kind="f32", rows=segs)
    assert np.isfinite(got["go"]).all() and np.isfinite(got["s0"]).all()
    ref = run_gdn(wl, final=True)
    np.testing.assert_array_equal(got["s0"].view(np.int32), ref["s0"].view(np.int32))
