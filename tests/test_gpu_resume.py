"""GPU parity of checkpoint resume: roots whose prefix keys and values come
from a cache filled by an earlier pass (the stream holds only new segments),
through fork_meta_build_ctx and fork_attn_forward_ctx, against the oracle,
against the plain tree in which each cached prefix is an explicit root
segment, and under a recorded graph."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, log
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def resumed_case(seed, dtype, n_seg, max_len, roots, H=8, Hkv=2, D=64, ctx_choices=(1, 63, 64, 65, 300)):
    """A random forest whose roots resume cached contexts (the second root
    shares the first's rows), q/k/v and the key/value cache; bf16 cases hold
    bf16-representable values."""
    rng = np.random.default_rng(seed)
    parent, seg_len = W.random_tree(rng, n_seg, max_len, max_depth=4, roots=roots)
    S = len(parent)
    rts = np.flatnonzero(parent < 0)
    cs, cl = np.zeros(S, np.int32), np.zeros(S, np.int32)
    rows = 0
    for i, r in enumerate(rts):
        if i == 1:
            cs[r], cl[r] = cs[rts[0]], cl[rts[0]]
            continue
        n = int(rng.choice(ctx_choices)) if i == 0 else int(rng.choice((0,) + tuple(ctx_choices)))
        cs[r], cl[r] = rows, n
        rows += n
    T = int(seg_len.sum())
    C = max(rows, 1)
    draw = lambda *shape: rng.standard_normal(shape).astype(np.float32)
    t = dict(q=draw(T, H, D), k=draw(T, Hkv, D), v=draw(T, Hkv, D), kc=draw(C, Hkv, D),
             vc=draw(C, Hkv, D))
    if dtype == "bf16":
        t = {k: W.round_bf16(v) for k, v in t.items()}
    return dict(parent=parent, seg_len=seg_len, ctx_start=cs, ctx_len=cl, C=C, T=T, S=S, H=H,
                Hkv=Hkv, D=D, dtype=dtype, **t)


def run_resume(c, split=True):
    caps = caps_for(c["parent"], c["seg_len"], c["H"] // c["Hkv"],
                    kv_heads=c["Hkv"] if split else 0, ctx_cap=c["C"])
    sess = ForkSession(**caps, D=c["D"])
    dt = TORCH_DT[c["dtype"]]
    dev = {k: torch.from_numpy(c[k]).to("cuda", dt) for k in ("q", "k", "v", "kc", "vc")}
    sess.build(c["parent"], c["seg_len"], ctx_start=c["ctx_start"], ctx_len=c["ctx_len"])
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((c["T"], c["H"]), float("nan"), device="cuda")
    sess.attention(dev["q"], dev["k"], dev["v"], o, lse, kc=dev["kc"], vc=dev["vc"])
    iso = np.zeros(c["T"], np.int32)
    B.fork_meta_export(sess.meta, B.ARR_TOK_ISO_POS, iso)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), iso


@pytest.mark.parametrize("dtype,D,seed", [("f32", 64, 1), ("bf16", 128, 2), ("bf16", 64, 3)])
def test_resume_parity(dtype, D, seed):
    c = resumed_case(seed, dtype, 12, 90, 3, D=D)
    log(f"resume {dtype} D={D}: T={c['T']} S={c['S']} contexts={c['ctx_len'][c['ctx_len'] > 0].tolist()}")
    ref_o, ref_lse = oracle.attention(c["parent"], c["seg_len"], c["q"], c["k"], c["v"],
                                      ctx_start=c["ctx_start"], ctx_len=c["ctx_len"], kc=c["kc"],
                                      vc=c["vc"])
    for split in (True, False):
        o, lse, iso = run_resume(c, split=split)
        check_close(f"resume.o split={split}", o, ref_o, dtype)
        check_close(f"resume.lse split={split}", lse, ref_lse, dtype, kind="f32")
    np.testing.assert_array_equal(iso, oracle.meta(c["parent"], c["seg_len"], c["ctx_len"])["tok_iso_pos"])


def test_resume_equals_plain_tree_on_gpu():
    """The resumed pass reproduces, on its new tokens, the pass over the plain
    tree that recomputes the cached prefix as an explicit root segment."""
    c = resumed_case(7, "bf16", 10, 80, 2, D=128)
    rts = np.flatnonzero(c["parent"] < 0)
    # plain tree: one segment per distinct nonempty range, then the forest
    ranges = sorted({(int(c["ctx_start"][r]), int(c["ctx_len"][r])) for r in rts if c["ctx_len"][r] > 0})
    rid = {x: i for i, x in enumerate(ranges)}
    nc = len(ranges)
    fp = np.array([-1] * nc + [(-1 if c["ctx_len"][s] == 0 else rid[(int(c["ctx_start"][s]), int(c["ctx_len"][s]))])
                               if c["parent"][s] < 0 else int(c["parent"][s]) + nc for s in range(c["S"])], np.int32)
    fl = np.array([n for _, n in ranges] + list(c["seg_len"]), np.int32)
    rows = [c0 + j for c0, n in ranges for j in range(n)]
    Tc = len(rows)
    H, Hkv, D = c["H"], c["Hkv"], c["D"]
    fq = np.concatenate([np.zeros((Tc, H, D), np.float32), c["q"]])
    fk = np.concatenate([c["kc"][rows], c["k"]])
    fv = np.concatenate([c["vc"][rows], c["v"]])
    sess = ForkSession(**caps_for(fp, fl, H // Hkv, kv_heads=Hkv), D=D)
    dq, dk, dv = (torch.from_numpy(x).to("cuda", torch.bfloat16) for x in (fq, fk, fv))
    sess.build(fp, fl)
    o = torch.full_like(dq, float("nan"))
    lse = torch.full((len(fq), H), float("nan"), device="cuda")
    sess.attention(dq, dk, dv, o, lse)
    torch.cuda.synchronize()
    full_o = o.float().cpu().numpy().astype(np.float64)[Tc:]
    full_lse = lse.cpu().numpy().astype(np.float64)[Tc:]
    ro, rlse, _ = run_resume(c)
    check_close("resume vs plain tree: o", ro, full_o, "bf16")
    check_close("resume vs plain tree: lse", rlse, full_lse, "bf16", kind="f32")


def test_resume_graph_replay():
    """A bucket with a context capacity, recorded once, replays resumed trees
    (and a tree with no context) as the eager calls compute them."""
    H, Hkv, D, GH, DK = 8, 2, 128, 2, 64
    T_CAP, S_CAP, C_CAP = 2048, 48, 1024
    sess = ForkSession(T_CAP, S_CAP, 4, H // Hkv, kv_heads=Hkv, D=D, gH=GH, dk=DK, dv=DK, ctx_cap=C_CAP)
    bf = torch.bfloat16
    buf = dict(q=torch.zeros(T_CAP, H, D, dtype=bf, device="cuda"),
               k=torch.zeros(T_CAP, Hkv, D, dtype=bf, device="cuda"),
               v=torch.zeros(T_CAP, Hkv, D, dtype=bf, device="cuda"),
               kc=torch.zeros(C_CAP, Hkv, D, dtype=bf, device="cuda"),
               vc=torch.zeros(C_CAP, Hkv, D, dtype=bf, device="cuda"),
               gq=torch.zeros(T_CAP, GH, DK, dtype=bf, device="cuda"),
               gk=torch.zeros(T_CAP, GH, DK, dtype=bf, device="cuda"),
               gv=torch.zeros(T_CAP, GH, DK, dtype=bf, device="cuda"),
               a=torch.ones(T_CAP, GH, device="cuda"), b=torch.zeros(T_CAP, GH, device="cuda"))
    o = torch.zeros(T_CAP, H, D, dtype=bf, device="cuda")
    lse = torch.zeros(T_CAP, H, device="cuda")
    go = torch.zeros(T_CAP, GH, DK, dtype=bf, device="cuda")
    s0 = torch.zeros(S_CAP, GH, DK, DK, device="cuda")
    cases = [resumed_case(s, "bf16", 10, 120, 2, H=H, Hkv=Hkv, D=D, ctx_choices=(5, 64, 300)) for s in (31, 32)]
    cases[1]["ctx_len"][:] = 0  # a tree without context in the same bucket
    first = True
    for c in cases:
        assert c["T"] <= T_CAP and c["S"] <= S_CAP and c["C"] <= C_CAP
        for n in ("q", "k", "v"):
            buf[n][:c["T"]].copy_(torch.from_numpy(c[n]).to(bf))
        for n in ("kc", "vc"):
            buf[n][:c[n].shape[0]].copy_(torch.from_numpy(c[n]).to(bf))
        # eager reference
        sess.build(c["parent"], c["seg_len"], ctx_start=c["ctx_start"], ctx_len=c["ctx_len"])
        eo = torch.full((c["T"], H, D), float("nan"), dtype=bf, device="cuda")
        else_ = torch.full((c["T"], H), float("nan"), device="cuda")
        sess.attention(buf["q"][:c["T"]], buf["k"][:c["T"]], buf["v"][:c["T"]], eo, else_,
                       kc=buf["kc"], vc=buf["vc"])
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            if first:
                sess.capture(dict(q=buf["q"], k=buf["k"], v=buf["v"], o=o, lse=lse, kc=buf["kc"], vc=buf["vc"]),
                             dict(q=buf["gq"], k=buf["gk"], v=buf["gv"], a=buf["a"], b=buf["b"], o=go,
                                  seg_start_state=s0))
                first = False
            sess.build(c["parent"], c["seg_len"], ctx_start=c["ctx_start"], ctx_len=c["ctx_len"])
            sess.replay()
        torch.cuda.synchronize()
        assert torch.equal(o[:c["T"]], eo), "graph replay differs from the eager call"
        assert torch.equal(lse[:c["T"]], else_)
        ref_o, _ = oracle.attention(c["parent"], c["seg_len"], c["q"], c["k"], c["v"],
                                    ctx_start=c["ctx_start"], ctx_len=c["ctx_len"], kc=c["kc"], vc=c["vc"])
        check_close("graph resume.o", o[:c["T"]].float().cpu().numpy().astype(np.float64), ref_o, "bf16")
    log("resume graph replay: 2 trees, replay == eager bitwise")


def test_agent_history_resume_sampled():
    """The benchmark's resumed agent history at full size (the 4096-token root
    cached and shared by its 8 children, now roots; 10,240 stream tokens),
    split tiles on as the benchmark runs it: sampled rows against the oracle,
    and the GDN layer resumed from the checkpointed state."""
    wl = W.agent_history()
    P = int(wl.seg_len[0])
    parent = (wl.parent[1:] - (wl.parent[1:] >= 0)).astype(np.int32)
    seg_len = wl.seg_len[1:].astype(np.int32)
    roots = parent < 0
    S, T = len(parent), int(seg_len.sum())
    cs, cl = np.zeros(S, np.int32), np.where(roots, P, 0).astype(np.int32)
    q, k, v = wl.q[P:], wl.k[P:], wl.v[P:]
    kc, vc = wl.k[:P], wl.v[:P]
    caps = caps_for(parent, seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv, ctx_cap=P)
    sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
    bf = torch.bfloat16
    dev = lambda x, dt=bf: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    sess.build(parent, seg_len, ctx_start=cs, ctx_len=cl)
    o = torch.full((T, wl.H, wl.D), float("nan"), dtype=bf, device="cuda")
    lse = torch.full((T, wl.H), float("nan"), device="cuda")
    sess.attention(dev(q), dev(k), dev(v), o, lse, kc=dev(kc), vc=dev(vc))
    # GDN: each new root starts from the checkpointed state (here the
    # workload's root state, the same for the 8 roots)
    R = int(roots.sum())
    rs = np.repeat(wl.root_state, R, axis=0)
    go = torch.full((T, wl.gH, wl.dv), float("nan"), dtype=bf, device="cuda")
    s0 = torch.full((S, wl.gH, wl.dv, wl.dk), float("nan"), device="cuda")
    sess.gdn(dev(wl.gq[P:]), dev(wl.gk[P:]), dev(wl.gv[P:]), dev(wl.a[P:], torch.float32),
             dev(wl.b[P:], torch.float32), go, s0, root_state=dev(rs, torch.float32))
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    st = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    picks = []
    for s in (0, 5, 7, 8, 100, 263):
        L = int(seg_len[s])
        picks += [st[s], st[s] + L - 1] + list(st[s] + rng.integers(0, L, 5))
    sel = np.zeros(T, np.uint8)
    sel[np.unique(picks)] = 1
    ref_o, ref_lse = oracle.attention(parent, seg_len, q, k, v, tok_select=sel, ctx_start=cs,
                                      ctx_len=cl, kc=kc, vc=vc)
    rows = sel.astype(bool)
    got_o = o.float().cpu().numpy().astype(np.float64)
    check_close("resume attn.o[sampled]", got_o, ref_o, "bf16", rows=rows)
    check_close("resume attn.lse[sampled]", lse.cpu().numpy().astype(np.float64), ref_lse, "bf16",
                kind="f32", rows=rows)
    assert np.isfinite(got_o).all()
    seg_pick = [0, 8, 263]
    ssel = np.zeros(S, np.uint8)
    ssel[seg_pick] = 1
    ref_go, ref_s0, _ = oracle.gdn(parent, seg_len, wl.gq[P:], wl.gk[P:], wl.gv[P:], wl.a[P:],
                                   wl.b[P:], root_state=rs, seg_select=ssel)
    trows = np.zeros(T, bool)
    for s in seg_pick:
        trows[st[s]:st[s] + seg_len[s]] = True
    check_close("resume gdn.o[sampled]", go.float().cpu().numpy().astype(np.float64), ref_go, "bf16",
                rows=trows)
    check_close("resume gdn.start_state[sampled]", s0.cpu().numpy().astype(np.float64), ref_s0, "bf16",
                kind="f32", rows=seg_pick)
