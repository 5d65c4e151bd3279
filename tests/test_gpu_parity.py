"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Covers the metadata (bit-exact), the dense tree mask (bit-exact), tree
attention and the forked Gated DeltaNet (within the stated tolerances) on
every parent array with up to 4 segments, ragged random trees spanning several
tiles and chunks, and the configured workloads (whole outputs where the oracle
is fast, sampled rows and segments at full size), plus run-to-run determinism.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, log, oracle_attn, oracle_gdn, run_hip
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

pytestmark = pytest.mark.gpu


def small_wl(parent, seg_len, dtype, seed, H=4, Hkv=2, D=64, gH=2, dk=32, root_std=None,
             gates="uniform"):
    return W.make_workload("case", dtype, parent, seg_len, H=H, Hkv=Hkv, D=D, gH=gH, dk=dk, dv=dk,
                           gates=gates, root_state_std=root_std, seed=seed)


def full_check(wl, attn=True, gdn=True):
    got = run_hip(wl, attn=attn, gdn=gdn)
    if attn:
        o, lse = oracle_attn(wl)
        check_close("attn.o", got["o"], o, wl.dtype)
        check_close("attn.lse", got["lse"], lse, wl.dtype, kind="f32")
    if gdn:
        go, s0, s1 = oracle_gdn(wl)
        check_close("gdn.o", got["go"], go, wl.dtype)
        check_close("gdn.start_state", got["s0"], s0, wl.dtype, kind="f32")
        check_close("gdn.final_state", got["s1"], s1, wl.dtype, kind="f32")
    return got


# ------------------------------------------------------------------ metadata

def _meta_case(parent, seg_len):
    parent = np.asarray(parent, np.int32)
    seg_len = np.asarray(seg_len, np.int32)
    caps = caps_for(parent, seg_len, 8)
    sess = ForkSession(**caps)
    meta = sess.build(parent, seg_len)
    torch.cuda.synchronize()
    ref = oracle.meta(parent, seg_len)
    T, S = int(seg_len.sum()), len(parent)
    for aid, key, n in ((B.ARR_TOK_SEG, "tok_seg", T), (B.ARR_TOK_POS, "tok_pos", T),
                        (B.ARR_TOK_ISO_POS, "tok_iso_pos", T), (B.ARR_SEG_START, "seg_start", S),
                        (B.ARR_DEPTH, "depth", S), (B.ARR_ANC_LEN, "anc_len", S),
                        (B.ARR_ROOT, "root", S)):
        dst = np.zeros(n, np.int32)
        B.fork_meta_export(meta, aid, dst)
        np.testing.assert_array_equal(dst, ref[key], err_msg=key)
    if T <= 4096:
        mask = torch.zeros((T, T), dtype=torch.uint8, device="cuda")
        B.fork_meta_dense_mask(meta, mask)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(mask.cpu().numpy(), oracle.mask(parent, seg_len))
    sess.close()


def test_meta_and_mask_bit_exact_small_trees():
    for S in range(1, 5):
        choices = [[-1]] + [list(range(-1, s)) for s in range(1, S)]
        for parent in itertools.product(*choices):
            for lens in ([1] * S, [3, 1, 2, 17][:S], [70, 2, 65, 1][:S]):
                _meta_case(parent, lens)


def test_meta_bit_exact_workload_trees():
    rng = np.random.Generator(np.random.PCG64(1005))
    for name, (parent, seg_len) in {
            "tiny": W.tree_one_level(32, [8] * 4),
            "one_request": W.tree_one_level(2048, list(range(16, 48, 2))),
            "wide": W.tree_one_level(8192, [8] * 256),
            "agent": W.tree_three_level(4096, 8, 512, 32, 24),
            "mix": W.request_mix_tree(rng)}.items():
        log(f"meta {name}")
        _meta_case(parent, seg_len)


# ----------------------------------------------------------------- tiny trees

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_small_trees(dtype):
    seed = 0
    for S in range(1, 5):
        choices = [[-1]] + [list(range(-1, s)) for s in range(1, S)]
        for parent in itertools.product(*choices):
            for lens in ([1, 2, 3, 1][:S], [17, 3, 1, 2][:S]):
                seed += 1
                p = np.array(parent, np.int32)
                log(f"case parent={parent} lens={lens} {dtype}")
                wl = small_wl(p, lens, dtype, seed, root_std=0.1)
                full_check(wl)


@pytest.mark.parametrize("dtype,D,dk,H,Hkv", [("f32", 64, 32, 4, 2), ("f32", 128, 64, 2, 2),
                                               ("bf16", 128, 128, 16, 2), ("bf16", 64, 64, 6, 3),
                                               ("bf16", 128, 32, 8, 1)])
def test_random_ragged_trees(dtype, D, dk, H, Hkv):
    """Ragged lengths spanning several 64-key tiles and 64-token chunks, multiple
    roots, depth up to 4, GQA groups that do and do not divide the tile."""
    rng = np.random.default_rng(D + dk + H)
    for trial in range(6):
        parent, seg_len = W.random_tree(rng, int(rng.integers(2, 10)), 150, max_depth=4,
                                        roots=int(rng.integers(1, 3)))
        log(f"ragged trial {trial}: S={len(parent)} T={int(seg_len.sum())} {dtype} D={D} dk={dk} "
            f"H={H}/{Hkv}")
        wl = W.make_workload("ragged", dtype, parent, seg_len, H=H, Hkv=Hkv, D=D, gH=3, dk=dk,
                             dv=dk, gates="sigmoid", root_state_std=0.1 if trial % 2 else None,
                             seed=1000 + trial)
        full_check(wl)


def test_long_segment_chain_ragged_tail():
    """A chain of long segments (several 64-chunks each, ragged tails)."""
    parent = np.array([-1, 0, 1, 2], np.int32)
    seg_len = np.array([301, 129, 64, 65], np.int32)
    wl = W.make_workload("chain", "bf16", parent, seg_len, H=8, Hkv=1, D=128, gH=2, dk=128,
                         dv=128, gates="sigmoid", root_state_std=None, seed=77)
    full_check(wl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deep_chain_past_planned_depths(dtype):
    """A path 40 segments deep (beyond the depths whose segment counts the
    host plans, so deeper launches split their depth from the blob), short
    segments mixed with multi-chunk ones, plus side branches."""
    rng = np.random.default_rng(40)
    n = 40
    parent = [-1] + list(range(n - 1))
    seg_len = list(rng.integers(3, 30, n))
    for d in (5, 20, 33, 38):
        seg_len[d] = int(rng.integers(65, 140))
    # side branches off deep segments
    for d in (10, 31, 35, 39):
        parent.append(d)
        seg_len.append(int(rng.integers(1, 90)))
    parent = np.array(parent, np.int32)
    seg_len = np.array(seg_len, np.int32)
    wl = W.make_workload("deep", dtype, parent, seg_len, H=4, Hkv=2, D=64, gH=2,
                         dk=64 if dtype == "bf16" else 32, dv=64 if dtype == "bf16" else 32,
                         gates="sigmoid", root_state_std=0.1, seed=4040)
    log(f"deep chain {dtype}: S={wl.S} T={wl.T} depth={n - 1}")
    full_check(wl)


@pytest.mark.parametrize("H,Hkv", [(32, 1), (64, 2), (3, 1), (128, 2), (256, 1)])
def test_large_and_odd_gqa_groups(H, Hkv):
    """GQA groups of 32, 64 and 128 query heads per kv head (8, 4 and 2 tokens
    per 256-row tile), 256 (the largest group: one token per tile) and 3 (rows
    not a multiple of the group)."""
    rng = np.random.default_rng(H * 7 + Hkv)
    for trial in range(2):
        parent, seg_len = W.random_tree(rng, 7, 120, max_depth=3, roots=1 + trial)
        wl = W.make_workload("gqa", "bf16", parent, seg_len, H=H, Hkv=Hkv, D=64, gH=2, dk=32,
                             dv=32, gates="sigmoid", root_state_std=None, seed=500 + trial)
        log(f"gqa {H}/{Hkv} trial {trial}: S={wl.S} T={wl.T}")
        full_check(wl, gdn=False)


def test_gdn_depth_split_mixed():
    """Depths that mix long segments (several chunks: the chunk-cooperative
    scan while they fit one round of workgroups) with short ones (the
    per-slice scan), two roots with a root state, ragged tails, a segment of
    exactly one chunk, and a third depth whose long segments are too many for
    the cooperative scan."""
    parent = np.array([-1, -1, 0, 0, 0, 1, 1, 2, 2, 2, 5, 5, 5], np.int32)
    seg_len = np.array([300, 150, 70, 30, 64, 129, 65, 200, 90, 3, 66, 130, 17], np.int32)
    for gH in (16, 4):
        log(f"depth split: gH={gH}")
        wl = W.make_workload("split", "bf16", parent, seg_len, H=8, Hkv=2, D=128, gH=gH, dk=128,
                             dv=128, gates="sigmoid", root_state_std=0.1, seed=4242 + gH)
        full_check(wl, attn=False)


# ---------------------------------------------------------------- workloads

def test_tiny_one_level_full():
    wl = W.tiny_one_level()
    full_check(wl)


def test_one_request_full():
    wl = W.one_request()
    got = full_check(wl)
    o_ref32 = oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, prec="f32")[0]
    fid = metrics.decision_fidelity(got["o"], o_ref32, wl.w_attn, wl.parent, wl.seg_len)
    log(f"  attention decision fidelity vs fp32 oracle: {fid}")
    g_ref32 = oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b, prec="f32")[0]
    fid = metrics.decision_fidelity(got["go"], g_ref32, wl.w_gdn, wl.parent, wl.seg_len)
    log(f"  GDN decision fidelity vs fp32 oracle: {fid}")
    assert fid["argmax_agreement"] == 1.0


def _sampled(wl, seg_pick, tok_pick, graph=False):
    """Full-size run, oracle on sampled tokens (attention) and segments (GDN)."""
    got = run_hip(wl)
    sel_t = np.zeros(wl.T, np.uint8)
    sel_t[tok_pick] = 1
    o, lse = oracle_attn(wl, tok_select=sel_t)
    rows = sel_t.astype(bool)
    check_close("attn.o[sampled]", got["o"], o, wl.dtype, rows=rows)
    check_close("attn.lse[sampled]", got["lse"], lse, wl.dtype, kind="f32", rows=rows)
    sel_s = np.zeros(wl.S, np.uint8)
    sel_s[seg_pick] = 1
    go, s0, s1 = oracle_gdn(wl, seg_select=sel_s)
    st = np.concatenate([[0], np.cumsum(wl.seg_len)[:-1]])
    trows = np.zeros(wl.T, bool)
    for s in seg_pick:
        trows[st[s]:st[s] + wl.seg_len[s]] = True
    check_close("gdn.o[sampled]", got["go"], go, wl.dtype, rows=trows)
    check_close("gdn.start_state[sampled]", got["s0"], s0, wl.dtype, kind="f32", rows=seg_pick)
    check_close("gdn.final_state[sampled]", got["s1"], s1, wl.dtype, kind="f32", rows=seg_pick)
    # every output is finite (nothing left unwritten)
    for k in ("o", "lse", "go", "s0", "s1"):
        assert np.isfinite(got[k]).all(), k


def _tok_sample(wl, segs, rng, per_seg=6):
    st = np.concatenate([[0], np.cumsum(wl.seg_len)[:-1]])
    picks = []
    for s in segs:
        L = int(wl.seg_len[s])
        picks += [st[s], st[s] + L - 1] + list(st[s] + rng.integers(0, L, per_seg))
    return np.unique(np.array(picks))


def test_wide_options_sampled():
    wl = W.wide_options()
    rng = np.random.default_rng(3)
    segs = [0, 1, 2, 128, 255, 256]
    _sampled(wl, [0, 1, 200, 256], _tok_sample(wl, segs, rng))


def test_agent_history_sampled():
    wl = W.agent_history()
    rng = np.random.default_rng(4)
    segs = [0, 1, 8, 9, 40, 264]
    _sampled(wl, [0, 3, 9, 100, 264], _tok_sample(wl, segs, rng))


def test_determinism_bitwise():
    wl = W.one_request()
    a = run_hip(wl)
    b = run_hip(wl)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_split_and_whole_tiles_agree():
    """Split query tiles (key-range parts merged by log-sum-exp) and whole tiles
    give the same attention within tolerance; both match the oracle."""
    wl = W.one_request()
    a = run_hip(wl, gdn=False, split=True)
    b = run_hip(wl, gdn=False, split=False)
    o, lse = oracle_attn(wl)
    check_close("split attn.o", a["o"], o, wl.dtype)
    check_close("whole attn.o", b["o"], o, wl.dtype)
    check_close("split attn.lse", a["lse"], lse, wl.dtype, kind="f32")
    check_close("whole attn.lse", b["lse"], lse, wl.dtype, kind="f32")


# ------------------------------------------------------------- fork copy

@pytest.mark.parametrize("name", ["one_request", "agent_history"])
def test_fork_copy_is_bitwise(name):
    """The fork writes the parent's end state into every child's start slot
    exactly: start[c] and final[parent[c]] agree bit for bit (fp32 words) on
    every child, at every depth (the three-level tree forks twice; its root
    starts from the given root state, copied bit for bit too)."""
    wl = W.WORKLOADS[name]()
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv)
    sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
    d = to_device(wl, "cuda")
    sess.build(wl.parent, wl.seg_len)
    go = torch.empty((wl.T, wl.gH, wl.dv), device="cuda", dtype=d["gq"].dtype)
    st0 = torch.full((wl.S, wl.gH, wl.dv, wl.dk), float("nan"), device="cuda")
    st1 = torch.full_like(st0, float("nan"))
    sess.gdn(d["gq"], d["gk"], d["gv"], d["a"], d["b"], go, st0, st1, root_state=d["root_state"])
    torch.cuda.synchronize()
    assert sess.check() == 0
    kids = torch.from_numpy(np.flatnonzero(wl.parent >= 0)).cuda()
    par = torch.from_numpy(wl.parent[wl.parent >= 0].astype(np.int64)).cuda()
    a = st0.index_select(0, kids).view(torch.int32)
    b = st1.index_select(0, par).view(torch.int32)
    assert torch.equal(a, b), "a child's start state differs from its parent's end state"
    roots = np.flatnonzero(wl.parent < 0)
    r0 = st0[torch.from_numpy(roots).cuda()]
    want = torch.zeros_like(r0) if d["root_state"] is None else d["root_state"]
    assert torch.equal(r0.view(torch.int32), want.contiguous().view(torch.int32))
    log(f"  {name}: {len(kids)} children start from their parent's end state, bit for bit")
    sess.close()
