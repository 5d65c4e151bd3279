"""The request mix (64 decision requests flattened into one stream, bf16,
attention 16/2/128, Gated DeltaNet 16 x 128 x 128) at full size, run the way
the benchmark runs it: replay of a graph recorded for its capacity bucket
(393,216 tokens x 4,096 segments, depth 1: a prefix with its options), on a
first tree and then on a second seed's tree built into the same bucket.

Checked against the oracle on sampled requests (the one with the longest
root, the one with the fewest and the one with the most options, and two
random ones): attention o and log-sum-exp on sampled rows of the root and the
first and last tokens of options; Gated DeltaNet o on every row of the root
and of three options, and their start and final states. Requests never see
each other, so the oracle runs on each sampled request alone (the inputs are
drawn per request, so they are the very values the stream holds). The fork
copy is checked bitwise on every child of the mix: its start state equals its
parent's final state exactly, and every root starts from zero. A second graph
of the same bucket, recorded without end states as the benchmark runs it
(leaf options then run packed, several to a chunk), is checked the same way
on the Gated DeltaNet (o and start states, and the fork copies bitwise equal
across siblings). On that graph, a property of the delta rule is checked on
every row of the mix without the oracle: with q = k, a = 1 and b = 1 / |k|^2,
every output row equals its value row."""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, log
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import (ForkSession, pick_bucket, pick_depth_cap,
                                                  request_mix_to_device)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SEEDS = (W.SEED_BASE + 5, W.SEED_BASE + 6)
H, HKV, D, GH, DK = 16, 2, 128, 16, 128


def threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def sample_requests(parent, seg_len, seed):
    spans = W.request_spans(parent, seg_len)
    roots = np.array([a for a, _, _, _ in spans])
    counts = np.array([b - a - 1 for a, b, _, _ in spans])
    rng = np.random.default_rng(seed)
    picks = [int(np.argmax(seg_len[roots])), int(np.argmin(counts)), int(np.argmax(counts))]
    picks += [int(x) for x in rng.choice(len(spans), 2, replace=False)]
    return list(dict.fromkeys(picks)), spans


@pytest.fixture(scope="module")
def bucket():
    """Session and device buffers of the bucket, the graph recorded once (on
    the first seed's tree, with final states)."""
    rng = np.random.Generator(np.random.PCG64(SEEDS[0]))
    parent, seg_len = W.request_mix_tree(rng)
    t_cap, s_cap = pick_bucket(int(seg_len.sum()), len(parent))
    assert (t_cap, s_cap) == (3 << 17, 1 << 12)
    sess = ForkSession(t_cap, s_cap, pick_depth_cap(1), H // HKV, kv_heads=HKV, D=D, gH=GH, dk=DK, dv=DK)
    log(f"bucket {t_cap} x {s_cap}: drawing seed {SEEDS[0]} (T={int(seg_len.sum())}, S={len(parent)})")
    _, _, t, _ = request_mix_to_device(SEEDS[0], t_cap, threads=threads())
    dev = "cuda"
    out = dict(o=torch.empty((t_cap, H, D), dtype=torch.bfloat16, device=dev),
               lse=torch.empty((t_cap, H), device=dev),
               go=torch.empty((t_cap, GH, DK), dtype=torch.bfloat16, device=dev),
               s0=torch.empty((s_cap, GH, DK, DK), device=dev),
               s1=torch.empty((s_cap, GH, DK, DK), device=dev))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sess.build(parent, seg_len)
        sess.capture(dict(q=t["q"], k=t["k"], v=t["v"], o=out["o"], lse=out["lse"]),
                     dict(q=t["gq"], k=t["gk"], v=t["gv"], a=t["a"], b=t["b"], o=out["go"],
                          seg_start_state=out["s0"], seg_final_state=out["s1"]))
    torch.cuda.synchronize()
    yield sess, t, out, stream
    sess.close()


def replay_seed(bucket, seed):
    sess, t, out, stream = bucket
    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = W.request_mix_tree(rng)
    log(f"seed {seed}: drawing T={int(seg_len.sum())} S={len(parent)} into the bucket")
    request_mix_to_device(seed, t["q"].shape[0], threads=threads(), out=t)
    for k in out:
        out[k].fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        sess.build(parent, seg_len)
        sess.replay()
    torch.cuda.synchronize()
    assert sess.check() == 0
    return parent, seg_len


def check_fork_bitwise(parent, out):
    """start[c] == final[parent[c]] bit for bit on every child; roots start at 0."""
    s0, s1 = out["s0"], out["s1"]
    kids = np.flatnonzero(parent >= 0)
    for i in range(0, len(kids), 256):
        c = torch.from_numpy(kids[i:i + 256]).cuda()
        p = torch.from_numpy(parent[kids[i:i + 256]].astype(np.int64)).cuda()
        a, b = s0.index_select(0, c), s1.index_select(0, p)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "fork copy differs from the parent's end state"
    roots = torch.from_numpy(np.flatnonzero(parent < 0)).cuda()
    assert torch.equal(s0.index_select(0, roots), torch.zeros_like(s0.index_select(0, roots)))
    log(f"  fork copy bitwise on {len(kids)} children; {len(roots)} roots start at zero")


def host(x, rows):
    return x[rows].float().cpu().numpy().astype(np.float64)


def check_requests(parent, seg_len, seed, out, attn=True, final=True):
    picks, spans = sample_requests(parent, seg_len, seed)
    for r in picks:
        a, b, t0, t1 = spans[r]
        wl = W.request_mix(seed, select=[r])
        n_opt = b - a - 1
        P = int(wl.seg_len[0])
        log(f"request {r}: root {P} tokens, {n_opt} options, stream rows [{t0}, {t1})")
        start = np.concatenate([[0], np.cumsum(wl.seg_len)[:-1]])
        rng = np.random.default_rng(seed * 1000 + r)
        opts = sorted(set([1, 2, n_opt - 1, n_opt] + [int(x) for x in rng.integers(1, n_opt + 1, 4)]))
        rows = list(range(min(16, P))) + list(range(P // 2, min(P, P // 2 + 16))) + list(range(max(0, P - 32), P))
        for c in opts:
            rows += [int(start[c]), int(start[c] + wl.seg_len[c] - 1)]
        rows = np.array(sorted(set(rows)))
        sel = np.zeros(wl.T, np.uint8)
        sel[rows] = 1
        if attn:
            o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, tok_select=sel)
            check_close(f"req {r} attn.o", host(out["o"], t0 + rows), o_ref[rows], "bf16")
            check_close(f"req {r} attn.lse", host(out["lse"], t0 + rows), lse_ref[rows], "bf16", kind="f32")
        gsegs = [0, 1, n_opt] if n_opt > 1 else [0, 1]
        gsegs = sorted(set(gsegs + [int(rng.integers(1, n_opt + 1))]))
        ssel = np.zeros(wl.S, np.uint8)
        ssel[gsegs] = 1
        go_ref, s0_ref, s1_ref = oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b,
                                            seg_select=ssel)
        trows = np.concatenate([np.arange(start[s], start[s] + wl.seg_len[s]) for s in gsegs])
        check_close(f"req {r} gdn.o (segments {gsegs})", host(out["go"], t0 + trows), go_ref[trows], "bf16")
        segs = np.array(gsegs)
        check_close(f"req {r} gdn.start_state", host(out["s0"], a + segs), s0_ref[segs], "bf16", kind="f32")
        if final:
            check_close(f"req {r} gdn.final_state", host(out["s1"], a + segs), s1_ref[segs], "bf16",
                        kind="f32")


def test_request_mix_full_size_graph_replay(bucket):
    parent, seg_len = replay_seed(bucket, SEEDS[0])
    check_fork_bitwise(parent, bucket[2])
    check_requests(parent, seg_len, SEEDS[0], bucket[2])


def test_request_mix_second_seed_same_bucket(bucket):
    parent, seg_len = replay_seed(bucket, SEEDS[1])
    check_fork_bitwise(parent, bucket[2])
    check_requests(parent, seg_len, SEEDS[1], bucket[2])


@pytest.fixture(scope="module")
def bucket_packed(bucket):
    """A second graph of the same bucket and inputs, recorded without end
    states, the way the benchmark runs the Gated DeltaNet: leaf siblings then
    run packed, several to a chunk."""
    _, t, _, stream = bucket
    rng = np.random.Generator(np.random.PCG64(SEEDS[0]))
    parent, seg_len = W.request_mix_tree(rng)
    t_cap, s_cap = pick_bucket(int(seg_len.sum()), len(parent))
    sess = ForkSession(t_cap, s_cap, pick_depth_cap(1), H // HKV, kv_heads=HKV, D=D, gH=GH, dk=DK, dv=DK)
    dev = "cuda"
    out = dict(o=torch.empty((t_cap, H, D), dtype=torch.bfloat16, device=dev),
               lse=torch.empty((t_cap, H), device=dev),
               go=torch.empty((t_cap, GH, DK), dtype=torch.bfloat16, device=dev),
               s0=torch.empty((s_cap, GH, DK, DK), device=dev))
    with torch.cuda.stream(stream):
        sess.build(parent, seg_len)
        sess.capture(dict(q=t["q"], k=t["k"], v=t["v"], o=out["o"], lse=out["lse"]),
                     dict(q=t["gq"], k=t["gk"], v=t["gv"], a=t["a"], b=t["b"], o=out["go"],
                          seg_start_state=out["s0"]))
    torch.cuda.synchronize()
    yield sess, t, out, stream
    sess.close()


def check_siblings_bitwise(parent, out):
    """Without end states: every child's start state equals, bit for bit, the
    start state of its parent's first child (where the parent's end state
    was written); roots start at zero."""
    s0 = out["s0"]
    kids = np.flatnonzero(parent >= 0)
    first = {}
    for c in kids:
        first.setdefault(int(parent[c]), int(c))
    for i in range(0, len(kids), 256):
        c = torch.from_numpy(kids[i:i + 256]).cuda()
        f = torch.from_numpy(np.array([first[int(parent[x])] for x in kids[i:i + 256]], np.int64)).cuda()
        assert torch.equal(s0.index_select(0, c).view(torch.int32), s0.index_select(0, f).view(torch.int32))
    roots = torch.from_numpy(np.flatnonzero(parent < 0)).cuda()
    assert torch.equal(s0.index_select(0, roots), torch.zeros_like(s0.index_select(0, roots)))
    log(f"  fork copies bitwise equal across siblings on {len(kids)} children")


def test_request_mix_packed_gdn_graph_replay(bucket_packed):
    parent, seg_len = replay_seed(bucket_packed, SEEDS[0])
    check_siblings_bitwise(parent, bucket_packed[2])
    check_requests(parent, seg_len, SEEDS[0], bucket_packed[2], attn=False, final=False)


def test_request_mix_gdn_reads_back_every_write(bucket_packed):
    """A property checked on every row of the mix, with no oracle: with q = k,
    a = 1 and b = 1 / |k|^2 the delta rule maps k_t to v_t whatever the state
    held (S_t k_t = S_{t-1}(k_t - k_t) + v_t), so every Gated DeltaNet output
    row equals its value row. Run in the benchmark's graph (packed leaves, no
    end states) over all 316,934 tokens and 16 heads: the bar is the output's
    half bf16 ulp + 2e-3 elementwise (the state's rows stay bounded under these
    projections, and the kernel's split bf16 products carry ~16 bits of them)."""
    sess, t, out, stream = bucket_packed
    parent, seg_len = replay_seed(bucket_packed, SEEDS[0])
    T = int(seg_len.sum())
    k = t["gk"][:T].float()
    t["gq"][:T].copy_(t["gk"][:T])
    t["a"][:T].fill_(1.0)
    t["b"][:T].copy_(1.0 / (k * k).sum(-1))
    for key in out:
        out[key].fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        sess.build(parent, seg_len)
        sess.replay()
    torch.cuda.synchronize()
    assert sess.check() == 0
    v = t["gv"][:T].float()
    err = (out["go"][:T].float() - v).abs()
    half_ulp = torch.exp2(torch.floor(torch.log2(v.abs().clamp_min(2.0**-126))) - 8)
    worst = float((err - half_ulp).max())
    log(f"  read-back over {T} tokens x {GH} heads: max |o - v| {float(err.max()):.3e}, "
        f"max excess over half an ulp {worst:.3e}")
    assert torch.isfinite(out["go"][:T].float()).all()
    assert worst <= 2e-3
