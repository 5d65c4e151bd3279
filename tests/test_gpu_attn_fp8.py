"""Tree attention with FP8 scores (fork_attn_forward_qk8) against the oracle,
through the C ABI. Queries and keys are quantised per (token, head) row to
E4M3 (the oracle's quantiser, bit-exact with the GPU's); the oracle runs the
exact attention on the decoded values (code x row scale) with the same bf16
values, so the comparison isolates the kernel's arithmetic: the parity bar is
the bf16 one (plain max-abs 2e-2 on o where |ref| < 8, 2e-2 on the
log-sum-exp). The cost of quantising itself is reported as the option
softmax's total-variation distance to the float32 oracle on the unquantised
inputs. The launch is also recorded once in a graph for a capacity bucket and
replayed on two trees, bit for bit against eager."""
import numpy as np
import pytest
import torch

import oracle
from oracle import mixer as OM
from tests.gpu_helpers import check_close, log
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for

pytestmark = pytest.mark.gpu


def quantize_rows(x):
    """E4M3 codes and scales of x [T, n, D] per (token, head) row."""
    T, n, D = x.shape
    codes, scale = OM.quantize_fp8(np.ascontiguousarray(x, np.float32).reshape(T * n, D))
    return codes.reshape(T, n, D), scale.astype(np.float32).reshape(T, n)


def decoded(codes, scale):
    T, n, D = codes.shape
    return OM.dequantize_fp8(codes.reshape(T * n, D), scale.reshape(T * n)).reshape(T, n, D).astype(np.float32)


def run_qk8(wl, sess, split=True):
    q8, qs = quantize_rows(wl.q)
    k8, ks = quantize_rows(wl.k)
    d = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    o = torch.full((wl.T, wl.H, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((wl.T, wl.H), float("nan"), device="cuda")
    sess.build(wl.parent, wl.seg_len)
    sess.attention_qk8(d(q8, torch.uint8), d(qs, torch.float32), d(k8, torch.uint8), d(ks, torch.float32),
                       d(wl.v, torch.bfloat16), o, lse)
    torch.cuda.synchronize()
    assert sess.check() == 0
    return (o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            decoded(q8, qs), decoded(k8, ks))


def session_for(wl, split=True):
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv if split else 0)
    return ForkSession(**caps, D=wl.D)


@pytest.mark.parametrize("seed,split", [(1, True), (2, False), (3, True), (4, True)])
def test_qk8_random_trees(seed, split):
    rng = np.random.default_rng(seed)
    parent, seg_len = W.random_tree(rng, int(rng.integers(3, 14)), int(rng.integers(20, 300)), max_depth=4,
                                    roots=int(rng.integers(1, 3)))
    wl = W.make_workload("qk8", "bf16", parent, seg_len, H=8 * (1 + seed % 2), Hkv=2, D=128, gH=1, dk=32, dv=32,
                         gates="sigmoid", root_state_std=None, seed=seed)
    sess = session_for(wl, split)
    o, lse, qd, kd = run_qk8(wl, sess)
    o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v)
    log(f"seed {seed}: T={wl.T} S={wl.S} H={wl.H} split={split}")
    check_close("qk8 o", o, o_ref, "bf16")
    check_close("qk8 lse", lse, lse_ref, "bf16", kind="f32")
    sess.close()


def test_qk8_one_request_full_and_fidelity():
    wl = W.one_request()
    sess = session_for(wl)
    o, lse, qd, kd = run_qk8(wl, sess)
    o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v)
    check_close("qk8 one_request o", o, o_ref, "bf16")
    check_close("qk8 one_request lse", lse, lse_ref, "bf16", kind="f32")
    o32 = oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, prec="f32")[0]
    fid = metrics.decision_fidelity(o, o32, wl.w_attn, wl.parent, wl.seg_len)
    log(f"  FP8 scores vs the float32 oracle on unquantised inputs: {fid}")
    assert fid["tvd_max"] <= 5e-2
    sess.close()


def test_qk8_agent_history_sampled():
    wl = W.agent_history()
    sess = session_for(wl)
    o, lse, qd, kd = run_qk8(wl, sess)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([rng.integers(0, wl.T, 300), [0, 4095, 4096, wl.T - 1]]))
    sel = np.zeros(wl.T, np.uint8)
    sel[rows] = 1
    o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v, tok_select=sel)
    check_close("qk8 agent_history o[sampled]", o, o_ref, "bf16", rows=rows)
    check_close("qk8 agent_history lse[sampled]", lse, lse_ref, "bf16", kind="f32", rows=rows)
    sess.close()


def test_qk8_graph_replay_two_trees():
    """FP8 scores recorded once in a graph for a capacity bucket with split
    tiles allowed (the launch and its merge pass read the tree from the blob),
    then replayed after each of two trees is built into the same blob: every
    replay equals the eager launch on that tree bit for bit (o and lse), with
    eager work and synchronisations between the replays."""
    t_cap, s_cap, depth_cap, H, Hkv, D = 4096, 64, 3, 16, 2, 128
    sess = ForkSession(t_cap, s_cap, depth_cap, H // Hkv, kv_heads=Hkv, D=D)
    wls = []
    for seed in (41, 42):
        rng = np.random.default_rng(seed)
        prefixes = rng.integers(300, 1200, 2)
        opts = [rng.integers(4, 33, int(rng.integers(2, 9))) for _ in range(2)]
        parent, seg_len = W.tree_requests(prefixes, opts)
        wls.append(W.make_workload("qk8_graph", "bf16", parent, seg_len, H=H, Hkv=Hkv, D=D, gH=1, dk=32, dv=32,
                                   gates="sigmoid", root_state_std=None, seed=seed))
        assert wls[-1].T <= t_cap and wls[-1].S <= s_cap
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    q8 = torch.zeros((t_cap, H, D), dtype=torch.uint8, device="cuda")
    k8 = torch.zeros((t_cap, Hkv, D), dtype=torch.uint8, device="cuda")
    qs, ks = torch.ones((t_cap, H), device="cuda"), torch.ones((t_cap, Hkv), device="cuda")
    v = torch.zeros((t_cap, Hkv, D), dtype=torch.bfloat16, device="cuda")
    o = torch.full((t_cap, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((t_cap, H), float("nan"), device="cuda")

    def load(wl):
        (c8, cs), (d8, ds) = quantize_rows(wl.q), quantize_rows(wl.k)
        q8[:wl.T].copy_(dev(c8, torch.uint8))
        qs[:wl.T].copy_(dev(cs, torch.float32))
        k8[:wl.T].copy_(dev(d8, torch.uint8))
        ks[:wl.T].copy_(dev(ds, torch.float32))
        v[:wl.T].copy_(dev(wl.v, torch.bfloat16))
        sess.build(wl.parent, wl.seg_len)

    def launch():
        sess.attention_qk8(q8, qs, k8, ks, v, o, lse)

    def snapshot(wl):
        torch.cuda.synchronize()
        return [x[:wl.T].float().cpu().numpy().copy() for x in (o, lse)]

    eager = []
    for wl in wls:
        load(wl)
        launch()
        eager.append(snapshot(wl))
        log(f"  tree T={wl.T} S={wl.S}: {sess.meta.num_attn_merges} split tiles")
    load(wls[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for rep, i in enumerate((0, 1, 0, 1)):
        load(wls[i])
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot(wls[i])
        for name, x, y in zip(("o", "lse"), got, eager[i]):
            np.testing.assert_array_equal(x.view(np.int32), y.view(np.int32), err_msg=f"replay {rep} {name}")
        log(f"  replay {rep} (tree {i}) equals the eager launch")
    wl = wls[1]
    qd, kd = decoded(*quantize_rows(wl.q)), decoded(*quantize_rows(wl.k))
    o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v)
    check_close("qk8 graph o", eager[1][0].astype(np.float64), o_ref, "bf16")
    check_close("qk8 graph lse", eager[1][1].astype(np.float64), lse_ref, "bf16", kind="f32")
    del graph
    sess.close()
