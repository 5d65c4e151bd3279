"""Host half of the library, CPU only: the C-ABI loads and exports every
declared symbol; the metadata plan matches the oracle's index arrays bit for
bit and its work lists satisfy their invariants; invalid input is rejected
before anything would be enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# header word indices of the blob (tree_structured_decision_amd/csrc/common.h)
H_NAMES = ["MAGIC", "T", "S", "R", "MAXDEPTH", "NTILES", "NCHUNKS", "TILE_TOKENS", "GQA",
           "OFF_PARENT", "OFF_SEGLEN", "OFF_SEGSTART", "OFF_DEPTH", "OFF_ROOT", "OFF_ROOTORD",
           "OFF_ANCLEN", "OFF_FIRSTCHILD", "OFF_CHUNKBASE", "OFF_LEVELOFF", "OFF_LEVELSEG",
           "OFF_CHUNKS", "OFF_TILES", "OFF_TOKSEG", "OFF_TOKPOS", "OFF_TOKISO", "UPLOAD_WORDS",
           "NMERGE", "OFF_MERGE", "NPARTS", "KV_HEADS", "OFF_LEVELLONG", "OFF_CTXSTART",
           "OFF_CTXLEN", "NCTX", "OFF_GDNREC", "OFF_GDNPACK", "OFF_PACKOFF"]
HI = {n: i for i, n in enumerate(H_NAMES)}
ATTN_ROWS = int(re.search(r"kAttnRows = (\d+);", open(os.path.join(
    ROOT, "tree_structured_decision_amd", "csrc", "common.h")).read()).group(1))


def test_header_indices_match_source():
    src = open(os.path.join(ROOT, "tree_structured_decision_amd", "csrc", "common.h")).read()
    body = src[src.index("enum MetaHeader"):src.index("MH_WORDS = 64")]
    names = re.findall(r"MH_([A-Z_]+)", body)
    assert names == H_NAMES


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "fork.h")).read()
    declared = set(re.findall(r"^(?:fork_status|const char\*)\s+(\w+)\(", header, re.M))
    assert declared == set(B.EXPORTS)
    L = B.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert B.fork_version().startswith("forkattn")


def plan(parent, seg_len, gqa=8, t_cap=None, s_cap=None, depth_cap=8, kv_heads=0, ctx=None,
         ctx_cap=None):
    """ctx: (ctx_start, ctx_len) int32 arrays of resumed contexts, or None."""
    parent = np.asarray(parent, np.int32)
    seg_len = np.asarray(seg_len, np.int32)
    if ctx_cap is None:
        ctx_cap = 0 if ctx is None else int((ctx[0] + ctx[1]).max(initial=0))
    caps = B.make_caps(t_cap or int(seg_len.sum()), s_cap or len(parent), depth_cap, gqa, kv_heads,
                       ctx_cap)
    _, stg = B.fork_meta_size(caps)
    staging = np.zeros(stg // 4, np.int32)
    if ctx is None:
        meta, up = B.fork_meta_plan(parent, seg_len, caps, staging)
    else:
        meta, up = B.fork_meta_plan_ctx(parent, seg_len, np.asarray(ctx[0], np.int32),
                                        np.asarray(ctx[1], np.int32), caps, staging)
    return meta, staging, up


def arr(w, name, n):
    off = w[HI["OFF_" + name]]
    return w[off:off + n]


def check_plan(parent, seg_len, gqa, kv_heads=0, ctx=None):
    parent = np.asarray(parent, np.int32)
    seg_len = np.asarray(seg_len, np.int32)
    meta, w, up = plan(parent, seg_len, gqa, kv_heads=kv_heads, ctx=ctx)
    S, T = len(parent), int(seg_len.sum())
    ctx_start = np.zeros(S, np.int32) if ctx is None else np.asarray(ctx[0], np.int32)
    ctx_len = np.zeros(S, np.int32) if ctx is None else np.asarray(ctx[1], np.int32)
    np.testing.assert_array_equal(arr(w, "CTXLEN", S), ctx_len)
    np.testing.assert_array_equal(arr(w, "CTXSTART", S), np.where(ctx_len > 0, ctx_start, 0))
    assert w[HI["NCTX"]] == int(np.sum(ctx_len > 0))
    assert w[HI["MAGIC"]] == 0x464B4D31
    assert (w[HI["T"]], w[HI["S"]]) == (T, S) == (meta.num_tokens, meta.num_segments)
    assert up == 4 * w[HI["UPLOAD_WORDS"]]
    ref = oracle.meta(parent, seg_len)
    np.testing.assert_array_equal(arr(w, "PARENT", S), parent)
    np.testing.assert_array_equal(arr(w, "SEGLEN", S), seg_len)
    for name, key in (("SEGSTART", "seg_start"), ("DEPTH", "depth"), ("ROOT", "root"),
                      ("ANCLEN", "anc_len")):
        np.testing.assert_array_equal(arr(w, name, S), ref[key], err_msg=name)
    # roots numbered in index order; first child = lowest-index child
    roots = np.flatnonzero(parent < 0)
    ro = arr(w, "ROOTORD", S)
    np.testing.assert_array_equal(ro[roots], np.arange(len(roots)))
    assert np.all(ro[parent >= 0] == -1)
    fc = arr(w, "FIRSTCHILD", S)
    for s in range(S):
        kids = np.flatnonzero(parent == s)
        assert fc[s] == (kids[0] if len(kids) else -1)
    # levels: a partition of the segments by depth, longest first
    maxd = int(ref["depth"].max())
    assert w[HI["MAXDEPTH"]] == maxd
    lo = arr(w, "LEVELOFF", maxd + 2)
    ls = arr(w, "LEVELSEG", S)
    assert sorted(ls.tolist()) == list(range(S))
    ll = arr(w, "LEVELLONG", maxd + 1)
    for d in range(maxd + 1):
        segs = ls[lo[d]:lo[d + 1]]
        assert np.all(ref["depth"][segs] == d)
        assert np.all(np.diff(seg_len[segs]) <= 0)
        # the depth's segments longer than one 64-token chunk lead its list
        assert ll[d] == int(np.sum(seg_len[segs] > 64))
        assert np.all(seg_len[segs[:ll[d]]] > 64) and np.all(seg_len[segs[ll[d]:]] <= 64)
    # the scan items' records, in level order: segment, first token, length,
    # the slot holding its start state (first child of its parent; -1 - root
    # ordinal for a root), first child
    rec = arr(w, "GDNREC", 8 * S).reshape(S, 8)
    first = {s: (np.flatnonzero(parent == s)[0] if np.any(parent == s) else -1) for s in range(S)}
    for i, s in enumerate(ls):
        src = first[parent[s]] if parent[s] >= 0 else -1 - int(np.flatnonzero(roots == s)[0])
        want = (s, ref["seg_start"][s], seg_len[s], src, first[s], 1, 0, 0)
        assert tuple(rec[i]) == want, (i, s, tuple(rec[i]), want)
    # the packed list: runs of consecutive leaf siblings of at most 64 tokens
    # in total share a record (greedily, in index order); every other segment
    # has its own; longest first within a depth, with the segments longer than
    # a chunk in the level list's order
    leaf = lambda s: parent[s] >= 0 and first[s] == -1 and seg_len[s] <= 64
    po = arr(w, "PACKOFF", maxd + 2)
    pk = arr(w, "GDNPACK", 8 * int(po[maxd + 1])).reshape(-1, 8)
    covered, pack_of = [], {}
    for d in range(maxd + 1):
        items = pk[po[d]:po[d + 1]]
        assert np.all(np.diff(items[:, 2]) <= 0)
        np.testing.assert_array_equal(items[:ll[d], 0], ls[lo[d]:lo[d] + ll[d]])
        for k, (s0, st, L, src, fc, nsib, p0, p1) in enumerate(items):
            segs = np.arange(s0, s0 + nsib)
            covered += segs.tolist()
            for s in segs:
                pack_of[int(s)] = (d, k)
            assert np.all(ref["depth"][segs] == d) and (p0, p1) == (0, 0)
            assert st == ref["seg_start"][s0] and L == seg_len[segs].sum()
            want_src = first[parent[s0]] if parent[s0] >= 0 else -1 - int(np.flatnonzero(roots == s0)[0])
            assert src == want_src
            if nsib > 1:
                assert L <= 64 and all(leaf(s) for s in segs) and np.all(parent[segs] == parent[s0])
            assert fc == (-1 if nsib > 1 else first[s0])
    assert sorted(covered) == list(range(S))
    for s in range(S - 1):
        if leaf(s) and leaf(s + 1) and parent[s] == parent[s + 1] and pack_of[s] != pack_of[s + 1]:
            d, k = pack_of[s]
            assert pk[po[d] + k][2] + seg_len[s + 1] > 64, "two joinable siblings left apart"
    # chunks: 64-token pieces of each segment, in order
    nch = w[HI["NCHUNKS"]]
    ch = arr(w, "CHUNKS", 2 * nch).reshape(-1, 2)
    cb = arr(w, "CHUNKBASE", S)
    for s in range(S):
        n = -(-int(seg_len[s]) // 64)
        got = ch[cb[s]:cb[s] + n]
        want = [(ref["seg_start"][s] + 64 * i, min(64, seg_len[s] - 64 * i)) for i in range(n)]
        np.testing.assert_array_equal(got, np.array(want).reshape(-1, 2))
    assert nch == sum(-(-int(L) // 64) for L in seg_len)
    # tiles: every token in exactly one query tile; tile tokens share one parent;
    # the entries of a tile cover its key-tile sequence [0, ktiles) exactly
    TT = w[HI["TILE_TOKENS"]]
    assert TT == max(1, ATTN_ROWS // gqa)
    nt = w[HI["NTILES"]]
    ent = arr(w, "TILES", 8 * nt).reshape(-1, 8)
    tok_seg = ref["tok_seg"]
    st = ref["seg_start"]
    # a tile's key tiles: its ancestors' ranges, its root's context, its own range
    anc_kt = np.zeros(S, np.int64)
    for s_ in range(S):
        if parent[s_] >= 0:
            anc_kt[s_] = anc_kt[parent[s_]] + -(-int(seg_len[parent[s_]]) // 64)
        else:
            anc_kt[s_] = -(-int(ctx_len[s_]) // 64)
    parts = {}
    for t0, t1, own_lo, info, kt0, kt1, slot, root in ent:
        assert root == ref["root"][tok_seg[t0]]
        parts.setdefault((t0, t1), []).append((kt0, kt1, slot))
    cover = np.zeros(T, np.int32)
    used_slots = []
    for (t0, t1), lst in parts.items():
        assert 0 <= t0 < t1 <= T and t1 - t0 <= TT
        cover[t0:t1] += 1
        segs = np.unique(tok_seg[t0:t1])
        assert len(set(parent[segs].tolist())) == 1
        if len(segs) > 1:
            assert np.all(parent[segs] >= 0) and np.all(seg_len[segs] < TT)
        kt = anc_kt[segs[0]] + -(-(t1 - st[tok_seg[t0]]) // 64)
        lst.sort()
        assert lst[0][0] == 0 and lst[-1][1] == kt
        for a_, b_ in zip(lst, lst[1:]):
            assert a_[1] == b_[0]
        if len(lst) == 1:
            assert lst[0][2] == -1
        else:
            used_slots += [x[2] for x in lst]
    for t0, t1, own_lo, info, kt0, kt1, slot, _ in ent:
        segs = np.unique(tok_seg[t0:t1])
        assert own_lo == st[tok_seg[t0]]
        assert (info & ((1 << 30) - 1)) == parent[segs[0]] + 1
        assert bool(info & (1 << 30)) == (len(segs) > 1)
    np.testing.assert_array_equal(cover, 1)
    costs = ent[:, 5] - ent[:, 4]
    assert np.all(np.diff(costs) <= 0), "work entries must be ordered most expensive first"
    # merge groups: consecutive partial slots, one group per split tile
    nm = w[HI["NMERGE"]]
    assert meta.num_attn_merges == nm
    mg = arr(w, "MERGE", 4 * nm).reshape(-1, 4)
    assert sorted(used_slots) == list(range(len(used_slots))) == list(range(w[HI["NPARTS"]]))
    for t0, t1, npart, slot0 in mg:
        lst = parts[(t0, t1)]
        assert len(lst) == npart and sorted(x[2] for x in lst) == list(range(slot0, slot0 + npart))
    assert w[HI["NPARTS"]] * max(kv_heads, 1) <= 2048
    if kv_heads == 0:
        assert nm == 0
    return nm
@pytest.mark.parametrize("name", ["tiny_one_level", "one_request", "wide_options",
                                  "agent_history"])
def test_plan_workload_trees(name):
    rng = np.random.default_rng(0)
    wl_tree = {"tiny_one_level": lambda: W.tree_one_level(32, [8] * 4),
               "one_request": lambda: W.tree_one_level(2048, rng.integers(16, 49, 16)),
               "wide_options": lambda: W.tree_one_level(8192, [8] * 256),
               "agent_history": lambda: W.tree_three_level(4096, 8, 512, 32, 24)}[name]
    parent, seg_len = wl_tree()
    for gqa in (1, 2, 8, 16):
        check_plan(parent, seg_len, gqa)
        check_plan(parent, seg_len, gqa, kv_heads=2)


def test_plan_splits_long_tiles_of_a_small_tree():
    """The one-request tree has too few query tiles for the GPU: long ones are
    split into key-range parts when kv_heads is given."""
    rng = np.random.default_rng(0)
    parent, seg_len = W.tree_one_level(2048, rng.integers(16, 49, 16))
    assert check_plan(parent, seg_len, 8, kv_heads=2) > 0
    assert check_plan(parent, seg_len, 8, kv_heads=0) == 0
    # a large tree needs no splitting
    parent, seg_len = W.tree_one_level(8192, [8] * 256)
    assert check_plan(parent, seg_len, 8, kv_heads=4) == 0


def test_plan_request_mix_tree():
    rng = np.random.Generator(np.random.PCG64(1005))
    parent, seg_len = W.request_mix_tree(rng)
    check_plan(parent, seg_len, 8)
    check_plan(parent, seg_len, 8, kv_heads=2)


def test_plan_random_trees():
    rng = np.random.default_rng(3)
    for _ in range(60):
        parent, seg_len = W.random_tree(rng, int(rng.integers(1, 30)), int(rng.integers(1, 90)),
                                        max_depth=5, roots=int(rng.integers(1, 4)))
        check_plan(parent, seg_len, int(rng.choice([1, 2, 3, 8, 16, 128])),
                   kv_heads=int(rng.choice([0, 1, 2, 8])))


def _status(fn):
    with pytest.raises(B.ForkError) as e:
        fn()
    return e.value.status


def test_plan_errors():
    ok_p, ok_l = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    assert _status(lambda: plan([0], [3])) == -2                 # parent not before child
    assert _status(lambda: plan([-1, 1], [3, 3])) == -2
    assert _status(lambda: plan([-1, -2], [3, 3])) == -2
    assert _status(lambda: plan([-1, 0], [3, 0])) == -2          # empty segment
    assert _status(lambda: plan([], [], t_cap=16, s_cap=4)) == -2  # no segments
    assert "at least one segment" in B.fork_last_error()
    assert _status(lambda: plan(ok_p, ok_l, t_cap=5)) == -5      # token capacity
    assert _status(lambda: plan(ok_p, ok_l, s_cap=1)) == -5      # segment capacity
    assert _status(lambda: plan([-1, 0, 1, 2], [1, 1, 1, 1], depth_cap=2)) == -5
    assert _status(lambda: plan(ok_p, ok_l, gqa=0)) == -3
    assert _status(lambda: plan(ok_p, ok_l, gqa=ATTN_ROWS + 1)) == -3
    caps = B.make_caps(6, 2, 2, 8)
    small = np.zeros(16, np.int32)
    assert _status(lambda: B.fork_meta_plan(ok_p, ok_l, caps, small)) == -4
    assert "staging" in B.fork_last_error()


def test_capacities_whose_blob_needs_over_2_31_words_are_rejected():
    """The header keeps int32 word offsets: capacities whose blob would reach
    2^31 words are refused at the size query (and so at every later call),
    not accepted with offsets that wrap."""
    assert _status(lambda: B.fork_meta_size(B.make_caps(1 << 29, 1 << 10, 4, ATTN_ROWS))) == -5
    assert "2^31" in B.fork_last_error()
    dev, _ = B.fork_meta_size(B.make_caps(1 << 20, 1 << 12, 4, 8))  # a large bucket still fits
    assert dev < (1 << 33)


def test_meta_check_argument_errors_without_gpu():
    """fork_meta_check validates its descriptor on the host before any HIP call."""
    assert _status(lambda: B.fork_meta_check(B.fork_meta(), stream=0)) == -1  # zero caps, no blob
    meta, _, _ = plan([-1, 0], [4, 2], gqa=2)
    assert meta.dev is None  # a plan has no device blob
    assert _status(lambda: B.fork_meta_check(meta, stream=0)) == -1
    assert "device blob" in B.fork_last_error()


def test_device_error_bits_match_header():
    """The binding's FORK_DEVERR_* values and FORK_E_DEVICE are the header's."""
    header = open(os.path.join(ROOT, "include", "fork.h")).read()
    assert int(re.search(r"#define FORK_DEVERR_MAGIC (\d+)", header).group(1)) == B.FORK_DEVERR_MAGIC
    assert int(re.search(r"#define FORK_DEVERR_CAPACITY (\d+)", header).group(1)) == B.FORK_DEVERR_CAPACITY
    assert int(re.search(r"FORK_E_DEVICE = (-\d+)", header).group(1)) == -7
    assert B.STATUS[-7] == "FORK_E_DEVICE"


def test_forward_argument_errors_without_gpu():
    """Argument errors come back before any HIP call, so they work on a host
    without a GPU (the device pointer below is never dereferenced)."""
    parent, seg_len = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    meta, _, _ = plan(parent, seg_len, gqa=2)
    dev_bytes, _ = B.fork_meta_size(meta.caps)
    meta.dev = 0x1000
    meta.dev_bytes = dev_bytes
    fake = 0x2000
    # unsupported head size / GQA mismatch / null tensors
    assert _status(lambda: B.fork_attn_forward(meta, fake, fake, fake, fake, None, 4, 2, 96, 0.0,
                                               B.FORK_BF16, stream=0)) == -3
    assert _status(lambda: B.fork_attn_forward(meta, fake, fake, fake, fake, None, 4, 1, 64, 0.0,
                                               B.FORK_BF16, stream=0)) == -1
    assert _status(lambda: B.fork_attn_forward(meta, None, fake, fake, fake, None, 4, 2, 64, 0.0,
                                               B.FORK_BF16, stream=0)) == -1
    assert _status(lambda: B.gdn_fork_forward(meta, fake, fake, fake, fake, fake, None, fake, fake,
                                              None, 2, 48, 48, 1.0, B.FORK_BF16, fake, 1 << 40,
                                              stream=0)) == -3
    need = B.gdn_fork_workspace(meta, 2, 32, 32, B.FORK_BF16)
    assert _status(lambda: B.gdn_fork_forward(meta, fake, fake, fake, fake, fake, None, fake, fake,
                                              None, 2, 32, 32, 1.0, B.FORK_BF16, fake, need - 1,
                                              stream=0)) == -4
    assert _status(lambda: B.gdn_fork_forward(meta, fake, fake, fake, fake, fake, None, fake, None,
                                              None, 2, 32, 32, 1.0, B.FORK_BF16, fake, need,
                                              stream=0)) == -1
    small = B.fork_meta()
    ctypes.memmove(ctypes.byref(small), ctypes.byref(meta), ctypes.sizeof(meta))
    small.dev_bytes = 16
    assert _status(lambda: B.fork_attn_forward(small, fake, fake, fake, fake, None, 4, 2, 64, 0.0,
                                               B.FORK_BF16, stream=0)) == -4
    assert _status(lambda: B.fork_meta_build(parent, seg_len, meta.caps, 0, np.zeros(4096, np.uint8),
                                             stream=0)) == -1


def forest_with_contexts(rng, parent, seg_len, shared=True):
    """Context ranges for the roots of a forest: fresh rows, and (shared) the
    second root naming the first root's rows."""
    parent = np.asarray(parent, np.int32)
    S = len(parent)
    cs, cl = np.zeros(S, np.int32), np.zeros(S, np.int32)
    rows = 0
    for i, r in enumerate(np.flatnonzero(parent < 0)):
        if shared and i == 1:
            cs[r], cl[r] = cs[np.flatnonzero(parent < 0)[0]], cl[np.flatnonzero(parent < 0)[0]]
            continue
        n = int(rng.choice([0, 1, 63, 64, 65, 300]))
        cs[r], cl[r] = rows, n
        rows += n
    return cs, cl


def test_plan_with_contexts():
    """Resumed contexts: the tiles of a root's tree count the context's key
    tiles, carry their root, and the blob holds the context ranges."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        parent, seg_len = W.random_tree(rng, int(rng.integers(1, 25)), int(rng.integers(1, 90)),
                                        max_depth=4, roots=int(rng.integers(1, 4)))
        ctx = forest_with_contexts(rng, parent, seg_len, shared=bool(rng.integers(0, 2)))
        gqa = int(rng.choice([1, 8, 16]))
        check_plan(parent, seg_len, gqa, ctx=ctx)
        check_plan(parent, seg_len, gqa, kv_heads=2, ctx=ctx)
    parent, seg_len = W.tree_three_level(64, 8, 512, 32, 24)
    check_plan(parent[1:] - (parent[1:] >= 0), seg_len[1:], 8, kv_heads=2,
               ctx=(np.zeros(len(parent) - 1, np.int32),
                    np.where(parent[1:] == 0, 4096, 0).astype(np.int32)))


def test_context_arguments_rejected():
    parent = np.array([-1, 0, -1], np.int32)
    seg_len = np.array([3, 2, 4], np.int32)
    z = np.zeros(3, np.int32)
    cases = [((z, np.array([0, 2, 0], np.int32)), B.ForkError, -2),      # context on a non-root
             ((z, np.array([-1, 0, 0], np.int32)), B.ForkError, -1),     # negative length
             ((np.array([0, 0, 9], np.int32), np.array([0, 0, 2], np.int32)), B.ForkError, -5)]  # past ctx_cap
    for ctx, exc, status in cases:
        with pytest.raises(exc) as e:
            plan(parent, seg_len, ctx=ctx, ctx_cap=10)
        assert e.value.status == status
    # one of the two arrays missing
    caps = B.make_caps(9, 3, 2, 8, 0, 10)
    _, stg = B.fork_meta_size(caps)
    staging = np.zeros(stg // 4, np.int32)
    with pytest.raises(B.ForkError) as e:
        B.fork_meta_plan_ctx(parent, seg_len, None, np.zeros(3, np.int32), caps, staging)
    assert e.value.status == -1
    # no context arrays: as fork_meta_plan
    meta, w, _ = plan(parent, seg_len, ctx=(z, z), ctx_cap=10)
    assert w[HI["NCTX"]] == 0


def test_resume_and_block_argument_errors_without_gpu():
    """The resume and block-piece entry points reject bad arguments before any
    HIP call (the device pointers below are never dereferenced)."""
    parent, seg_len = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    fake = 0x2000

    def fake_meta(ctx_cap):
        meta, _, _ = plan(parent, seg_len, gqa=2, ctx=(np.zeros(2, np.int32), np.zeros(2, np.int32)),
                          ctx_cap=ctx_cap)
        meta.dev = 0x1000
        meta.dev_bytes = B.fork_meta_size(meta.caps)[0]
        return meta

    m0, m1 = fake_meta(0), fake_meta(64)
    # a context capacity needs the cache; none forbids one
    assert _status(lambda: B.fork_attn_forward(m1, fake, fake, fake, fake, None, 4, 2, 64, 0.0,
                                               B.FORK_BF16, stream=0)) == -1
    assert _status(lambda: B.fork_attn_forward_ctx(m0, fake, fake, fake, fake, fake, fake, None, 4, 2,
                                                   64, 0.0, B.FORK_BF16, stream=0)) == -1
    # rotary embedding: head size, theta, null input
    assert _status(lambda: B.fork_rope_forward(m0, fake, 2, 12, 10000.0, B.FORK_BF16, stream=0)) == -3
    assert _status(lambda: B.fork_rope_forward(m0, fake, 2, 64, 1.0, B.FORK_BF16, stream=0)) == -1
    assert _status(lambda: B.fork_rope_forward(m0, None, 2, 64, 10000.0, B.FORK_BF16, stream=0)) == -1
    # convolution: channels, width, activation, in place, misaligned weights
    conv = lambda C=16, K=4, act=1, x=fake, w=fake, y=0x3000: _status(
        lambda: B.fork_conv_forward(m0, x, w, None, None, y, C, K, act, B.FORK_BF16, stream=0))
    assert conv(C=12) == -3
    assert conv(K=9) == -3 and conv(K=1) == -3
    assert conv(act=2) == -1
    assert conv(y=fake) == -1
    assert conv(w=fake + 4) == -1


def test_mixer_piece_argument_errors_without_gpu():
    """The gate, Gated DeltaNet input and projection entry points reject bad
    arguments before any HIP call (device pointers are never dereferenced)."""
    parent, seg_len = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    meta, _, _ = plan(parent, seg_len, gqa=2)
    meta.dev = 0x1000
    meta.dev_bytes = B.fork_meta_size(meta.caps)[0]
    fake = 0x2000
    gate = lambda mode=1, g=fake, w=fake, D=64, nh=2, eps=1e-6, dt=B.FORK_BF16, ld=0: _status(
        lambda: B.fork_gate_forward(meta, fake, g, w, 0x3000, nh, D, mode, eps, dt, stream=0, ld_g=ld))
    assert gate(ld=100) == -1 and gate(ld=132) == -1   # below nheads * D / not a multiple of 8
    assert gate(g=fake + 8) == -1                      # misaligned gate
    assert gate(mode=3) == -1 and gate(mode=-1) == -1
    assert gate(mode=0, g=None) == -1 and gate(mode=1, g=None) == -1
    assert gate(mode=1, w=None) == -1 and gate(mode=2, w=None) == -1
    assert gate(w=fake + 4) == -1
    assert gate(D=12) == -3 and gate(D=0) == -3
    assert gate(nh=0) == -1
    assert gate(eps=0.0) == -1
    assert gate(dt=7) == -3
    gi = lambda H=2, dk=64, dv=64, eps=1e-6, q=fake: _status(
        lambda: B.gdn_inputs_forward(meta, fake, fake, fake, fake, q, fake, fake, fake, fake, H, dk, dv,
                                     eps, B.FORK_BF16, stream=0))
    assert gi(q=None) == -1
    assert gi(H=0) == -1
    assert gi(dk=12) == -3 and gi(dv=2048) == -3
    assert gi(eps=-1.0) == -1
    assert _status(lambda: B.gdn_inputs_forward(meta, fake, fake, fake, fake, fake, fake, fake, fake, fake, 2, 64, 64,
                                                1e-6, B.FORK_BF16, stream=0, ld_ab=3)) == -1
    lin = lambda M=4, N=8, K=16, x=fake, y=0x3000, acc=0, dt=B.FORK_BF16: _status(
        lambda: B.fork_linear_forward(x, 0x4000, y, M, N, K, acc, dt, stream=0))
    assert lin(acc=2) == -1
    assert lin(M=0) == -1 and lin(K=-1) == -1
    assert lin(x=None) == -1
    assert lin(y=fake) == -1
    assert lin(dt=9) == -3


def test_fp8_argument_errors_without_gpu():
    fake = 0x2000
    qz = lambda rows=4, K=64, x=fake, q=0x3000, dt=B.FORK_BF16: _status(
        lambda: B.fork_quantize_fp8(x, q, 0x4000, rows, K, dt, stream=0))
    assert qz(rows=0) == -1 and qz(x=None) == -1
    assert qz(K=12) == -3 and qz(K=0) == -3
    assert qz(x=fake + 8) == -1 and qz(q=0x3004) == -1
    assert qz(dt=5) == -3
    lf = lambda M=4, N=8, K=64, acc=0, y=0x5000: _status(
        lambda: B.fork_linear_fp8_forward(fake, 0x3000, 0x4000, 0x4800, y, M, N, K, acc, stream=0))
    assert lf(K=24) == -3
    assert lf(M=0) == -1 and lf(acc=3) == -1
    assert lf(y=fake) == -1


def test_rope_copy_argument_errors_without_gpu():
    parent, seg_len = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    meta, _, _ = plan(parent, seg_len, gqa=2)
    meta.dev = 0x1000
    meta.dev_bytes = B.fork_meta_size(meta.caps)[0]
    rc = lambda src=0x10000, ld=256, dst=0x80000, nh=2, D=128, theta=10000.0, dt=B.FORK_BF16: _status(
        lambda: B.fork_rope_copy_forward(meta, src, ld, dst, nh, D, theta, dt, stream=0))
    assert rc(ld=255) == -1 and rc(ld=254) == -1   # below nheads * D / not a multiple of 4
    assert rc(D=12) == -3
    assert rc(theta=0.5) == -1
    assert rc(src=0x10002) == -1                   # misaligned
    assert rc(dst=0x10000 + 512) == -1             # overlapping
    assert rc(src=None) == -1


def test_conv_inputs_argument_errors_without_gpu():
    parent, seg_len = np.array([-1, 0], np.int32), np.array([4, 2], np.int32)
    meta, _, _ = plan(parent, seg_len, gqa=2)
    meta.dev = 0x1000
    meta.dev_bytes = B.fork_meta_size(meta.caps)[0]
    f = 0x2000
    ci = lambda H=2, dk=64, dv=64, K=4, eps=1e-6, w=0x3000, q=0x4000: _status(
        lambda: B.gdn_conv_inputs_forward(meta, f, w, None, None, q, 0x5000, 0x6000, H, dk, dv, K, eps,
                                          B.FORK_BF16, stream=0))
    assert ci(dk=64, dv=32) == -3 and ci(dk=48, dv=48) == -3 and ci(dk=1024, dv=1024) == -3
    assert ci(K=9) == -3 and ci(K=1) == -3
    assert ci(w=0x3004) == -1 and ci(eps=0.0) == -1 and ci(H=0) == -1
    assert ci(q=f) == -1 and ci(q=None) == -1
    # gdn_inputs without c needs only ab, the gate parameters and a, b
    assert _status(lambda: B.gdn_inputs_forward(meta, None, f, 0x3000, 0x4000, None, None, None, None, 0x5000,
                                                2, 64, 64, 1e-6, B.FORK_BF16, stream=0)) == -1  # a is null


def test_option_readout_argument_errors_without_gpu():
    """The decision readout rejects bad arguments before any HIP call (device
    pointers are never dereferenced)."""
    parent, seg_len = np.array([-1, 0, 0], np.int32), np.array([4, 2, 3], np.int32)
    meta, _, _ = plan(parent, seg_len, gqa=2)
    meta.dev = 0x1000
    meta.dev_bytes = B.fork_meta_size(meta.caps)[0]
    fake = 0x2000
    ro = lambda x=fake, w=fake, C=64, score=0x3000, prob=0x4000, dt=B.FORK_BF16: _status(
        lambda: B.fork_option_readout(meta, x, w, C, score, prob, dt, stream=0))
    assert ro(x=None) == -1 and ro(w=None) == -1 and ro(score=None) == -1 and ro(prob=None) == -1
    assert ro(C=12) == -3 and ro(C=0) == -3 and ro(C=65544) == -3
    assert ro(x=fake + 8) == -1 and ro(w=fake + 4) == -1
    assert ro(dt=7) == -3
