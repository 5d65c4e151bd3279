"""Gated DeltaNet with FP8 inputs (gdn_fork_forward_fp8) against the oracle,
through the C ABI. q, k and v are quantised per (token, head) row to E4M3 by
the oracle's quantiser (bit-exact with the GPU's); the oracle runs the exact
forked recurrence on the decoded values (code x row scale), so the comparison
isolates the kernel's arithmetic and the bar is the bf16 one (plain max-abs
2e-2 on o where |ref| < 8; 2e-2 on the fp32 start and end states). Cases:
random trees of several depths and roots with given root states, with and
without end states (without them, leaf siblings run packed); a long root that
the bf16 path would give to the chunk-cooperative kernel; the one-request
tree at full size; the fork copies bit for bit (every child's start state is
its parent's end state); the FP8 launch against the bf16 launch on the decoded
inputs where those are exact in bf16 (unit scales: the two differ only in the
order the matrix cores sum the products Q K^T and K K^T); and the host
rejections; and the launch recorded once in a graph for a capacity bucket,
replayed on two trees bit for bit against the eager launch. The cost of
quantising is reported as the option softmax's
total-variation distance to the float32 oracle on the unquantised inputs."""
import numpy as np
import pytest
import torch

import oracle
from oracle import mixer as OM
from tests.gpu_helpers import check_close, log
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

pytestmark = pytest.mark.gpu


def quantize_rows(x):
    """E4M3 codes and scales of x [T, n, D] per (token, head) row."""
    T, n, D = x.shape
    codes, scale = OM.quantize_fp8(np.ascontiguousarray(x, np.float32).reshape(T * n, D))
    return codes.reshape(T, n, D), scale.astype(np.float32).reshape(T, n)


def decoded(codes, scale):
    T, n, D = codes.shape
    return OM.dequantize_fp8(codes.reshape(T * n, D), scale.reshape(T * n)).reshape(T, n, D).astype(np.float32)


def session_for(wl):
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv)
    return ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)


def run_fp8(wl, sess, final, quant=None):
    """The FP8 launch on the workload's Gated DeltaNet inputs, quantised (or
    the given (codes, scales) triples); returns outputs and decoded inputs."""
    if quant is None:
        quant = [quantize_rows(x) for x in (wl.gq, wl.gk, wl.gv)]
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    (q8, qs), (k8, ks), (v8, vs) = quant
    d = to_device(wl, "cuda")
    sess.build(wl.parent, wl.seg_len)
    go = torch.full((wl.T, wl.gH, wl.dv), float("nan"), device="cuda", dtype=torch.bfloat16)
    st0 = torch.full((wl.S, wl.gH, wl.dv, wl.dk), float("nan"), device="cuda")
    st1 = torch.full_like(st0, float("nan")) if final else None
    sess.gdn_fp8(dev(q8, torch.uint8), dev(qs, torch.float32), dev(k8, torch.uint8), dev(ks, torch.float32),
                 dev(v8, torch.uint8), dev(vs, torch.float32), d["a"], d["b"], go, st0, st1,
                 root_state=d["root_state"])
    torch.cuda.synchronize()
    assert sess.check() == 0
    out = {"go": go, "s0": st0}
    if final:
        out["s1"] = st1
    res = {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}
    return res, [decoded(c, s) for c, s in quant]


def oracle_on(wl, qkv, seg_select=None):
    return oracle.gdn(wl.parent, wl.seg_len, qkv[0], qkv[1], qkv[2], wl.a, wl.b, root_state=wl.root_state,
                      seg_select=seg_select)


def check_forks(wl, got):
    p = np.asarray(wl.parent)
    kids = np.flatnonzero(p >= 0)
    s0 = got["s0"].astype(np.float32)[kids]
    s1 = got["s1"].astype(np.float32)[p[kids]]
    np.testing.assert_array_equal(s0.view(np.int32), s1.view(np.int32))


@pytest.mark.parametrize("seed,roots,final", [(21, 1, True), (22, 3, False), (23, 2, True), (24, 2, False)])
def test_fp8_gdn_random_trees(seed, roots, final):
    rng = np.random.default_rng(seed)
    parent, seg_len = W.random_tree(rng, int(rng.integers(4, 24)), int(rng.integers(20, 200)), max_depth=4,
                                    roots=roots)
    wl = W.make_workload("gdn8", "bf16", parent, seg_len, H=2, Hkv=2, D=64, gH=3, dk=128, dv=128,
                         gates="sigmoid" if seed % 2 else "uniform",
                         root_state_std=0.5 if roots > 1 else None, seed=seed)
    sess = session_for(wl)
    got, qkv = run_fp8(wl, sess, final)
    go, s0, s1 = oracle_on(wl, qkv)
    log(f"seed {seed}: T={wl.T} S={wl.S} roots={roots} end states={final}")
    check_close("gdn8.o", got["go"], go, "bf16")
    check_close("gdn8.start_state", got["s0"], s0, "bf16", kind="f32")
    if final:
        check_close("gdn8.final_state", got["s1"], s1, "bf16", kind="f32")
        check_forks(wl, got)
    sess.close()


def test_fp8_gdn_long_root_and_packed_leaves():
    """A 1,000-token root (16 chunks, on the fused kernel here) with 40 short
    leaves, without end states (the leaves run packed)."""
    rng = np.random.default_rng(25)
    parent = np.array([-1] + [0] * 40, np.int32)
    seg_len = np.array([1000] + list(rng.integers(1, 30, 40)), np.int32)
    wl = W.make_workload("gdn8_long", "bf16", parent, seg_len, H=2, Hkv=2, D=64, gH=4, dk=128, dv=128,
                         gates="sigmoid", root_state_std=None, seed=25)
    sess = session_for(wl)
    got, qkv = run_fp8(wl, sess, final=False)
    go, s0, _ = oracle_on(wl, qkv)
    check_close("gdn8_long.o", got["go"], go, "bf16")
    check_close("gdn8_long.start_state", got["s0"], s0, "bf16", kind="f32")
    sess.close()


def test_fp8_gdn_unit_scales_match_bf16_launch():
    """Rows whose largest |value| is 448 quantise with scale 1, so their
    decoded values are the codes, exact in bf16, and the factors are 1 (b
    kappa^2 = b, nu / kappa = 1, rho = 1): the FP8 launch and the bf16 launch
    on those values compute the same recurrence with the same bf16 operands,
    except that Q K^T and K K^T come from the FP8 matrix cores (exact
    products, fp32 sums in another order). They agree to that rounding: o
    within one bf16 ulp or 1e-4 of its largest magnitude, states within 1e-4
    of their largest magnitude: the codes reach 448, and a last-bit difference
    in a product moves the hi / lo bf16 split of the next operand, whose
    precision is about 2^-16.
    Segments of at most one chunk, so that the bf16 launch also runs every
    segment on the fused kernel."""
    rng = np.random.default_rng(26)
    parent, seg_len = W.random_tree(rng, 16, 64, max_depth=3, roots=2)
    wl = W.make_workload("gdn8_unit", "bf16", parent, seg_len, H=2, Hkv=2, D=64, gH=2, dk=128, dv=128,
                         gates="sigmoid", root_state_std=0.3, seed=26)
    quant = []
    for x in (wl.gq, wl.gk, wl.gv):
        # every row's maximum |value| is 448: scale 1, codes = nearest E4M3 values
        y = np.asarray(x, np.float32) * 60.0
        y[..., 0] = 448.0
        codes, scale = quantize_rows(y)
        assert np.all(scale == 1.0)
        quant.append((codes, scale))
    qkv = [decoded(c, s) for c, s in quant]
    # the same tensors through the bf16 entry point
    wl.gq, wl.gk, wl.gv = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in qkv)
    # (|k|^2 is now about 448^2: scale b so that b |k|^2 stays below 1)
    wl.b = (np.asarray(wl.b, np.float32) * np.float32(1.0 / 448.0 ** 2)).astype(np.float32)
    sess = session_for(wl)
    got8, _ = run_fp8(wl, sess, final=True, quant=quant)
    d = to_device(wl, "cuda")
    sess.build(wl.parent, wl.seg_len)
    go = torch.full((wl.T, wl.gH, wl.dv), float("nan"), device="cuda", dtype=torch.bfloat16)
    st0 = torch.full((wl.S, wl.gH, wl.dv, wl.dk), float("nan"), device="cuda")
    st1 = torch.full_like(st0, float("nan"))
    sess.gdn(d["gq"], d["gk"], d["gv"], d["a"], d["b"], go, st0, st1, root_state=d["root_state"])
    torch.cuda.synchronize()
    assert sess.check() == 0
    assert int(np.max(wl.seg_len)) <= 64
    for name, a8, ab in (("o", got8["go"], go), ("start", got8["s0"], st0), ("final", got8["s1"], st1)):
        ab = ab.float().cpu().numpy().astype(np.float64)
        err = np.abs(a8 - ab)
        if name == "o":
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ab), 1e-30))) - 7)
            bad = err > np.maximum(ulp * 1.0001, 1e-4 * np.abs(ab).max())
            same = float(np.mean(err == 0))
            log(f"  unit scales, FP8 vs bf16 launch, o: {same:.4f} of values equal, max difference "
                f"{err.max():.2e} (largest |o| {np.abs(ab).max():.2e})")
        else:
            bad = err > 1e-4 * np.abs(ab).max()
            log(f"  unit scales, FP8 vs bf16 launch, {name} state: max difference {err.max():.2e} "
                f"(largest |state| {np.abs(ab).max():.2e})")
        assert not bad.any(), name
    # (o reaches ~900 here, beyond what the absolute bf16 bar is for; the states stay O(1))
    _, s0_ref, s1_ref = oracle_on(wl, qkv)
    check_close("gdn8_unit.start_state", got8["s0"], s0_ref, "bf16", kind="f32")
    check_close("gdn8_unit.final_state", got8["s1"], s1_ref, "bf16", kind="f32")
    sess.close()


def test_fp8_gdn_one_request_full_and_fidelity():
    wl = W.one_request()
    sess = session_for(wl)
    got, qkv = run_fp8(wl, sess, final=True)
    go, s0, s1 = oracle_on(wl, qkv)
    check_close("gdn8 one_request o", got["go"], go, "bf16")
    check_close("gdn8 one_request start_state", got["s0"], s0, "bf16", kind="f32")
    check_close("gdn8 one_request final_state", got["s1"], s1, "bf16", kind="f32")
    check_forks(wl, got)
    o32 = oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b, prec="f32")[0]
    fid = metrics.decision_fidelity(got["go"], o32, wl.w_gdn, wl.parent, wl.seg_len)
    log(f"  FP8 inputs vs the float32 oracle on unquantised inputs: {fid}")
    assert fid["tvd_max"] <= 5e-2
    sess.close()


def test_fp8_gdn_rejections():
    wl = W.one_request()
    sess = session_for(wl)
    sess.build(wl.parent, wl.seg_len)
    T, H = wl.T, wl.gH
    z8 = torch.zeros((T, H, 128), dtype=torch.uint8, device="cuda")
    sc = torch.ones((T, H), device="cuda")
    ab = torch.full((T, H), 0.5, device="cuda")
    o = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((wl.S, H, 128, 128), device="cuda")
    with pytest.raises(B.ForkError) as e:
        B.gdn_fork_forward_fp8(sess.meta, z8, sc, z8, sc, z8, sc, ab, ab, None, o, st, None, H, 64, 64, 1.0)
    assert e.value.status == -3  # FORK_E_UNSUPPORTED
    with pytest.raises(B.ForkError) as e:
        B.gdn_fork_forward_fp8(sess.meta, z8, None, z8, sc, z8, sc, ab, ab, None, o, st, None, H, 128, 128, 1.0)
    assert e.value.status == -1  # FORK_E_ARG
    with pytest.raises(B.ForkError) as e:
        B.gdn_fork_forward_fp8(sess.meta, z8.data_ptr() + 1, sc, z8, sc, z8, sc, ab, ab, None, o, st, None, H, 128,
                               128, 1.0)
    assert e.value.status == -1  # (q8 not 16-byte aligned)
    sess.close()


def test_fp8_gdn_graph_replay_two_trees():
    """The FP8 launch recorded once in a graph for a capacity bucket (every
    depth up to the bucket's, the tree read from the blob), then replayed after
    each of two trees is built into the same blob: every replay equals the
    eager launch on that tree bit for bit (o, start and end states), with
    eager work and synchronisations between the replays."""
    t_cap, s_cap, depth_cap, gH = 3072, 96, 3, 4
    sess = ForkSession(t_cap, s_cap, depth_cap, 1, D=64, gH=gH, dk=128, dv=128)
    wls = []
    for seed in (31, 32):
        rng = np.random.default_rng(seed)
        parent, seg_len = W.random_tree(rng, int(rng.integers(20, 60)), 90, max_depth=4, roots=2)
        wls.append(W.make_workload("gdn8_graph", "bf16", parent, seg_len, H=1, Hkv=1, D=64, gH=gH, dk=128,
                                   dv=128, gates="sigmoid", root_state_std=0.5, seed=seed))
        assert wls[-1].T <= t_cap and wls[-1].S <= s_cap
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    # bucket-sized inputs and outputs, filled per tree
    q8, k8, v8 = (torch.zeros((t_cap, gH, 128), dtype=torch.uint8, device="cuda") for _ in range(3))
    qs, ks, vs = (torch.ones((t_cap, gH), device="cuda") for _ in range(3))
    a, b = torch.ones((t_cap, gH), device="cuda"), torch.zeros((t_cap, gH), device="cuda")
    root = torch.zeros((2, gH, 128, 128), device="cuda")
    go = torch.full((t_cap, gH, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    s0 = torch.full((s_cap, gH, 128, 128), float("nan"), device="cuda")
    s1 = torch.full_like(s0, float("nan"))

    def load(wl):
        for (codes, sc), dst, dsc in zip([quantize_rows(x) for x in (wl.gq, wl.gk, wl.gv)], (q8, k8, v8),
                                         (qs, ks, vs)):
            dst[:wl.T].copy_(dev(codes, torch.uint8))
            dsc[:wl.T].copy_(dev(sc, torch.float32))
        a[:wl.T].copy_(dev(wl.a, torch.float32))
        b[:wl.T].copy_(dev(wl.b, torch.float32))
        root.copy_(dev(wl.root_state, torch.float32))
        sess.build(wl.parent, wl.seg_len)

    def launch():
        sess.gdn_fp8(q8, qs, k8, ks, v8, vs, a, b, go, s0, s1, root_state=root)

    def snapshot(wl):
        torch.cuda.synchronize()
        return [x[:n].float().cpu().numpy().copy() for x, n in ((go, wl.T), (s0, wl.S), (s1, wl.S))]

    eager = []
    for wl in wls:
        load(wl)
        launch()
        eager.append(snapshot(wl))
    load(wls[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for rep, i in enumerate((0, 1, 0, 1)):
        load(wls[i])
        go.fill_(float("nan"))
        s0.fill_(float("nan"))
        s1.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot(wls[i])
        for name, x, y in zip(("o", "start", "final"), got, eager[i]):
            np.testing.assert_array_equal(x.view(np.int32), y.view(np.int32), err_msg=f"replay {rep} {name}")
        log(f"  replay {rep} (tree {i}: T={wls[i].T} S={wls[i].S}) equals the eager launch")
    go_ref, s0_ref, s1_ref = oracle_on(wls[1], [decoded(*quantize_rows(x)) for x in (wls[1].gq, wls[1].gk,
                                                                                      wls[1].gv)])
    check_close("gdn8 graph o", eager[1][0].astype(np.float64), go_ref, "bf16")
    check_close("gdn8 graph final_state", eager[1][2].astype(np.float64), s1_ref, "bf16", kind="f32")
    del graph
    sess.close()
