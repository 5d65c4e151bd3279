"""Graph buckets on the GPU: a recorded graph of both layers, replayed after
new trees are built into the same capacity bucket."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import check_close, log, oracle_attn, oracle_gdn
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession

pytestmark = pytest.mark.gpu

T_CAP, S_CAP, DEPTH_CAP = 4096, 64, 3
H, HKV, D, GH, DK = 16, 2, 128, 4, 128


def bucket_tensors():
    dev = "cuda"
    bf = torch.bfloat16
    t = dict(q=torch.zeros(T_CAP, H, D, dtype=bf, device=dev),
             k=torch.zeros(T_CAP, HKV, D, dtype=bf, device=dev),
             v=torch.zeros(T_CAP, HKV, D, dtype=bf, device=dev),
             gq=torch.zeros(T_CAP, GH, DK, dtype=bf, device=dev),
             gk=torch.zeros(T_CAP, GH, DK, dtype=bf, device=dev),
             gv=torch.zeros(T_CAP, GH, DK, dtype=bf, device=dev),
             a=torch.ones(T_CAP, GH, device=dev), b=torch.zeros(T_CAP, GH, device=dev))
    out = dict(o=torch.full((T_CAP, H, D), float("nan"), dtype=bf, device=dev),
               lse=torch.full((T_CAP, H), float("nan"), device=dev),
               go=torch.full((T_CAP, GH, DK), float("nan"), dtype=bf, device=dev),
               s0=torch.full((S_CAP, GH, DK, DK), float("nan"), device=dev),
               s1=torch.full((S_CAP, GH, DK, DK), float("nan"), device=dev))
    return t, out


def fill(t, wl):
    T = wl.T
    for name, src in (("q", wl.q), ("k", wl.k), ("v", wl.v), ("gq", wl.gq), ("gk", wl.gk),
                      ("gv", wl.gv), ("a", wl.a), ("b", wl.b)):
        t[name][:T].copy_(torch.from_numpy(src).to(t[name].dtype))


def make_tree_wl(seed, n_req):
    rng = np.random.default_rng(seed)
    prefixes = rng.integers(100, 600, n_req)
    opts = [rng.integers(4, 33, int(rng.integers(2, 9))) for _ in range(n_req)]
    parent, seg_len = W.tree_requests(prefixes, opts)
    return W.make_workload("graph", "bf16", parent, seg_len, H=H, Hkv=HKV, D=D, gH=GH, dk=DK, dv=DK,
                           gates="sigmoid", root_state_std=None, seed=seed)


def np64(x, n):
    return x[:n].float().cpu().numpy().astype(np.float64)


def test_graph_replay_matches_eager_and_oracle():
    sess = ForkSession(T_CAP, S_CAP, DEPTH_CAP, H // HKV, kv_heads=HKV, D=D, gH=GH, dk=DK, dv=DK)
    t, out = bucket_tensors()
    wa = make_tree_wl(1, 3)
    assert wa.T <= T_CAP and wa.S <= S_CAP
    fill(t, wa)
    # eager reference on tree A
    sess.build(wa.parent, wa.seg_len)
    eo = torch.full_like(out["o"], float("nan"))
    else_ = torch.full_like(out["lse"], float("nan"))
    ego = torch.full_like(out["go"], float("nan"))
    es0 = torch.full_like(out["s0"], float("nan"))
    es1 = torch.full_like(out["s1"], float("nan"))
    sess.attention(t["q"][:wa.T], t["k"][:wa.T], t["v"][:wa.T], eo, else_)
    sess.gdn(t["gq"][:wa.T], t["gk"][:wa.T], t["gv"][:wa.T], t["a"][:wa.T], t["b"][:wa.T], ego, es0, es1)
    torch.cuda.synchronize()
    # record the graph (built for tree A), replay
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sess.capture(dict(q=t["q"], k=t["k"], v=t["v"], o=out["o"], lse=out["lse"]),
                     dict(q=t["gq"], k=t["gk"], v=t["gv"], a=t["a"], b=t["b"], o=out["go"],
                          seg_start_state=out["s0"], seg_final_state=out["s1"]))
        sess.build(wa.parent, wa.seg_len)
        sess.replay()
    torch.cuda.synchronize()
    for k, e in (("o", eo), ("lse", else_), ("go", ego)):
        np.testing.assert_array_equal(np64(out[k], wa.T), np64(e, wa.T), err_msg=k)
        assert torch.isnan(out[k][wa.T:].float()).all(), f"{k}: rows past T were written"
    for k, e in (("s0", es0), ("s1", es1)):
        np.testing.assert_array_equal(np64(out[k], wa.S), np64(e, wa.S), err_msg=k)
    log("graph replay == eager (bitwise) on tree A")

    # new trees into the same bucket; eager torch work between replays
    for seed, n_req in ((2, 4), (3, 2), (4, 4)):
        wb = make_tree_wl(seed, n_req)
        assert wb.T <= T_CAP and wb.S <= S_CAP
        fill(t, wb)
        for k in out:
            out[k].fill_(float("nan"))
        with torch.cuda.stream(stream):
            sess.build(wb.parent, wb.seg_len)
            sess.replay()
        torch.cuda.synchronize()
        _ = (t["q"].float() * 2).sum().item()  # unrelated eager work between replays
        log(f"tree seed={seed}: T={wb.T} S={wb.S}")
        o, lse = oracle_attn(wb)
        check_close("graph attn.o", np64(out["o"], wb.T), o, "bf16")
        check_close("graph attn.lse", np64(out["lse"], wb.T), lse, "bf16", kind="f32")
        go, s0, s1 = oracle_gdn(wb)
        check_close("graph gdn.o", np64(out["go"], wb.T), go, "bf16")
        check_close("graph gdn.start", np64(out["s0"], wb.S), s0, "bf16", kind="f32")
        check_close("graph gdn.final", np64(out["s1"], wb.S), s1, "bf16", kind="f32")
    sess.close()
