"""Benchmark of the ForkAttention hot path on one MI355X.

A step is one pass of the whole path over one batch of decision requests:
segment metadata build (host plan, one upload from pinned memory, per-token
expansion kernel) and both layers, tree attention then the forked Gated
DeltaNet. The headline workload is the request mix: 64 decision requests
flattened into one stream (prefix lengths 1/P on 256..16384, option counts
1/n on 2..256, option lengths U{4..32}; bf16; attention 16 q / 2 kv heads x
128, Gated DeltaNet 16 heads x 128 x 128), padded into a capacity bucket of
393,216 tokens x 4,096 segments and run as replay of a graph recorded once
for that bucket. Inputs are the seeded PCG64 draws the parity tests check,
resident in HBM before the timed region. `value` is stream tokens per second
(every physical token counted once).

Also reported on the same JSON line:
  roofline      the dominant kernel (tree attention, fork_attn_kernel): its
                algorithmic flops per launch over its mean launch time (HIP
                events on its stream, an eager pass of the same tree) against
                the bf16 MFMA peak; roofline_gdn the same for the Gated
                DeltaNet layer against HBM;
  cpu_baseline  the float32 oracle on a prefix of the mix's requests (about
                15 s of work on every core of this host);
  fidelity      total-variation distance of per-option softmax scores of
                those requests against the float32 oracle;
  layers        per-layer P50 / P95 / mean (eager) and the graph replay's;
  workloads     all five workloads (and the resumed agent history), eager and
                graph replay, P50 / P95, per-layer roofline fractions;
  rates         option tokens/s, isolated-equivalent tokens/s, us per option;
  readout       the decision readout on the GPU (per-option scores and
                per-group probabilities of the whole tree), its time per call
                and its distance to the host float64 readout of the same rows;
  measured_peaks  a bf16 GEMM and a device copy on this GPU;
  block_ops, mixers, stack  the hybrid-block pieces, mixers and a four-layer
                stack on the one-request tree.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "branch tokens/s for ForkAttention + GDN fork layer; % of HBM/MFMA roofline"
PEAK_BF16_MFMA = 2.5e15      # dense, FLOP/s
PEAK_FP8_MFMA = 5.0e15
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12            # B/s
SEED_MIXER = 2048             # seed of the mixer weights and input
CPU_BUDGET_S = 15.0           # CPU-baseline sample: about this much oracle work


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_sha256() -> str:
    """Hash of every native source (kernels, host plan, public header): the
    counter runs stand only for the code they were taken on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_structured_decision_amd", "csrc")
    for f in sorted(os.listdir(csrc)) + ["../../include/fork.h"]:
        path = os.path.join(csrc, f)
        if os.path.isfile(path):
            h.update(f.encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per call of `kernel` on `workload` from the committed counter
    runs (profiles/hbm_traffic.json), or None when any native source has
    changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[workload][kernel]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if rec.get("sources_sha256") != sources_sha256():
        return None
    return dict(bytes=rec["read_bytes"] + rec["write_bytes"], read=rec["read_bytes"],
                write=rec["write_bytes"], summary=rec["summary"])


# ------------------------------------------------------------ algorithmic work

def visible_pairs(parent, seg_len, ctx_len=None) -> int:
    """Sum over tokens of (ancestor tokens + resumed context of the root +
    position in segment + 1)."""
    parent = np.asarray(parent)
    seg_len = np.asarray(seg_len, np.int64)
    anc = np.zeros(len(parent), np.int64)
    for s in range(len(parent)):
        if parent[s] >= 0:
            anc[s] = anc[parent[s]] + seg_len[parent[s]]
        elif ctx_len is not None:
            anc[s] = int(ctx_len[s])
    return int(np.sum(anc * seg_len + seg_len * (seg_len + 1) // 2))


def attn_work(parent, seg_len, H, Hkv, D, elt, ctx_len=None, ctx_rows=0):
    """Algorithmic flops (4 D H per visible pair) and bytes (q, k, v, o of the
    stream, plus the cached context's k, v read once)."""
    T = int(np.sum(seg_len))
    flops = 4.0 * D * H * visible_pairs(parent, seg_len, ctx_len)
    bytes_ = float(T * (2 * H + 2 * Hkv) * D * elt + ctx_rows * 2 * Hkv * D * elt)
    return flops, bytes_


def gdn_work(parent, seg_len, H, dk, dv, elt, root_state: bool):
    """Algorithmic bytes: q, k, v, o of the stream and a, b (fp32), every
    child's start state written once (the fork copy: S - R states), and the
    roots' given states read once when there are any."""
    T = int(np.sum(seg_len))
    S = len(parent)
    R = int(np.sum(np.asarray(parent) < 0))
    io = T * H * ((2 * dk + 2 * dv) * elt + 8)
    fork = (S - R) * H * dk * dv * 4
    rs = R * H * dk * dv * 4 if root_state else 0
    return float(io + fork + rs)


def tree_rates(parent, seg_len):
    """Option (leaf) count, option tokens and isolated-equivalent tokens (sum
    over leaves of the leaf's root-to-leaf path length: what per-branch
    recompute would process)."""
    parent = np.asarray(parent)
    seg_len = np.asarray(seg_len, np.int64)
    S = len(parent)
    anc = np.zeros(S, np.int64)
    has_child = np.zeros(S, bool)
    for s in range(S):
        if parent[s] >= 0:
            anc[s] = anc[parent[s]] + seg_len[parent[s]]
            has_child[parent[s]] = True
    leaves = ~has_child
    return int(leaves.sum()), int(seg_len[leaves].sum()), int((anc + seg_len)[leaves].sum())


def measured_peaks():
    """Achievable peaks on this GPU: a bf16 8192^3 GEMM (the vendor library,
    dense) and a 1 GiB device-to-device copy."""
    import torch

    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * 8192 ** 3 * n / (e0.elapsed_time(e1) * 1e-3)
    del a, b
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * (1 << 30) * n / (e0.elapsed_time(e1) * 1e-3)  # read + write bytes
    del src, dst
    return dict(bf16_gemm_tflops=gemm / 1e12, copy_gbs=copy / 1e9)



# ------------------------------------------------------------------ runners

def depth_of(parent):
    parent = np.asarray(parent)
    d = np.zeros(len(parent), np.int64)
    for s in range(len(parent)):
        if parent[s] >= 0:
            d[s] = d[parent[s]] + 1
    return int(d.max())


def wl_meta_of(parent, seg_len, H, Hkv, D, gH, dk, dv, dtype="bf16"):
    return dict(parent=np.asarray(parent, np.int32), seg_len=np.asarray(seg_len, np.int32),
                T=int(np.sum(seg_len)), S=len(parent), depth=depth_of(parent), H=H, Hkv=Hkv, D=D,
                gH=gH, dk=dk, dv=dv, dtype=dtype)


class Runner:
    """Device buffers and one step of the path for one workload. graph: the
    session is sized for the workload's capacity bucket and both layers are
    recorded once into a graph; a step then builds the tree into the blob and
    replays. Eager steps (also possible on a graph runner) launch both layers
    directly, each launch sized from the host plan."""

    def __init__(self, wl_meta: dict, tensors: dict, graph: bool):
        import torch
        from tree_structured_decision_amd.session import ForkSession, pick_bucket, pick_depth_cap

        self.m = wl_meta
        self.t = tensors
        T, S = wl_meta["T"], wl_meta["S"]
        depth = wl_meta["depth"]
        if graph:
            t_cap, s_cap = pick_bucket(T, S)
            depth_cap = pick_depth_cap(depth)
        else:
            t_cap, s_cap, depth_cap = T, S, depth
        self.caps = (t_cap, s_cap, depth_cap)
        self.ctx = wl_meta.get("ctx")  # (ctx_start, ctx_len, cache rows) of a resumed tree
        self.sess = ForkSession(t_cap, s_cap, depth_cap, wl_meta["H"] // wl_meta["Hkv"],
                                kv_heads=wl_meta["Hkv"], D=wl_meta["D"],
                                gH=wl_meta["gH"], dk=wl_meta["dk"], dv=wl_meta["dv"],
                                ctx_cap=0 if self.ctx is None else self.ctx[2])
        dev = "cuda"
        qd = tensors["q"].dtype
        H, D, gH, dv, dk = wl_meta["H"], wl_meta["D"], wl_meta["gH"], wl_meta["dv"], wl_meta["dk"]
        if graph:  # inputs must span the bucket's rows
            for n in ("q", "k", "v", "gq", "gk", "gv", "a", "b"):
                x = tensors[n]
                if x.shape[0] < t_cap:
                    y = torch.zeros((t_cap,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
                    y[:x.shape[0]].copy_(x)
                    tensors[n] = y
        self.o = torch.empty((t_cap, H, D), dtype=qd, device=dev)
        self.lse = torch.empty((t_cap, H), dtype=torch.float32, device=dev)
        self.go = torch.empty((t_cap, gH, dv), dtype=qd, device=dev)
        self.st0 = torch.empty((s_cap, gH, dv, dk), dtype=torch.float32, device=dev)
        self.graph = graph
        self.build()
        if graph:
            t = tensors
            self.sess.capture(dict(q=t["q"], k=t["k"], v=t["v"], o=self.o, lse=self.lse,
                                   kc=t.get("kc"), vc=t.get("vc")),
                              dict(q=t["gq"], k=t["gk"], v=t["gv"], a=t["a"], b=t["b"],
                                   root_state=t.get("root_state"), o=self.go,
                                   seg_start_state=self.st0))

    def build(self):
        if self.ctx is None:
            self.sess.build(self.m["parent"], self.m["seg_len"])
        else:
            self.sess.build(self.m["parent"], self.m["seg_len"], ctx_start=self.ctx[0],
                            ctx_len=self.ctx[1])

    def step(self, ev=None, eager=False):
        """One step; ev: three events recorded before attention, between the
        layers (eager only) and after the Gated DeltaNet."""
        t = self.t
        self.build()
        if self.graph and not eager:
            if ev:
                ev[0].record()
            self.sess.replay()
            if ev:
                ev[2].record()
            return
        if ev:
            ev[0].record()
        self.sess.attention(t["q"], t["k"], t["v"], self.o, self.lse, kc=t.get("kc"), vc=t.get("vc"))
        if ev:
            ev[1].record()
        self.sess.gdn(t["gq"], t["gk"], t["gv"], t["a"], t["b"], self.go, self.st0,
                      root_state=t.get("root_state"))
        if ev:
            ev[2].record()

    def close(self):
        self.sess.close()


def stats_us(xs_ms):
    x = np.asarray(xs_ms, np.float64) * 1e3
    return dict(p50_us=float(np.percentile(x, 50)), p95_us=float(np.percentile(x, 95)),
                mean_us=float(x.mean()))


def time_runner(r: Runner, steps: int, warmup: int, eager: bool, evict=None):
    """Times `steps` steps after `warmup`, twice: first plain steps between two
    synchronisations (the wall time per step: nothing else is enqueued), then
    the same number of steps with HIP events on the launch stream around each
    layer (eager) or around the replay (graph): an event record costs a few
    microseconds of GPU time, so this pass is not the one the wall time
    comes from. evict: a large device buffer written before every step of the
    event pass (outside the events) so that the inputs come from HBM rather
    than the L2 / Infinity Cache; then the wall pass is skipped."""
    import torch

    for _ in range(warmup):
        r.step(eager=eager)
    torch.cuda.synchronize()
    wall = None
    if evict is None:
        t0 = time.perf_counter()
        for _ in range(steps):
            r.step(eager=eager)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        if evict is not None:
            evict.fill_(k & 0xff)
        r.step(evs[k], eager=eager)
    torch.cuda.synchronize()
    if wall is None:
        wall = time.perf_counter() - t0
    out = dict(ms_per_step=wall / steps * 1e3)
    if eager:
        attn = [e[0].elapsed_time(e[1]) for e in evs]
        gdn = [e[1].elapsed_time(e[2]) for e in evs]
        out["attention"] = stats_us(attn)
        out["gdn"] = stats_us(gdn)
        out["pair"] = stats_us([a + g for a, g in zip(attn, gdn)])
    else:
        out["pair"] = stats_us([e[0].elapsed_time(e[2]) for e in evs])
    return out


def tensors_from_numpy(wl):
    from tree_structured_decision_amd.session import to_device

    return to_device(wl, "cuda")


def fp8_scores(r: Runner, meta, steps, warmup):
    """Tree attention with FP8 scores (E4M3 q and k with per-row scales on the
    FP8 matrix cores, bf16 values) on the runner's tree: the row quantisation
    runs once outside the timed launches (HIP events on the launch stream,
    eager). Returns the timing and the output (for the fidelity check)."""
    import torch

    t = r.t
    T, H, D, Hkv = meta["T"], meta["H"], meta["D"], meta["Hkv"]
    q8, qs = r.sess.quantize_fp8(t["q"][:T].reshape(T * H, D))
    k8, ks = r.sess.quantize_fp8(t["k"][:T].reshape(T * Hkv, D))
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), device="cuda")
    r.build()
    run = lambda: r.sess.attention_qk8(q8.view(T, H, D), qs.view(T, H), k8.view(T, Hkv, D), ks.view(T, Hkv),
                                       t["v"], o, lse)
    for _ in range(warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    fl = attn_work(meta["parent"], meta["seg_len"], H, Hkv, D, 2)[0]
    qk_share = 0.5  # QK^T and PV have equal flops: half at the fp8 peak, half at the bf16 peak
    roof = fl * qk_share / PEAK_FP8_MFMA + fl * (1 - qk_share) / PEAK_BF16_MFMA
    return dict(p50_us=st["p50_us"], p95_us=st["p95_us"], mean_us=st["mean_us"],
                achieved_tflops=fl / (st["mean_us"] * 1e-6) / 1e12, roofline_frac=roof / (st["mean_us"] * 1e-6),
                note="fork_attn_forward_qk8, eager; roofline: QK^T flops at the fp8 peak (5.0 PFLOP/s), PV flops at "
                     "the bf16 peak; fidelity against the float32 oracle on the unquantised inputs is in "
                     "fidelity.attention_fp8_scores", o=o)


def fp8_gdn(r: Runner, meta, steps, warmup):
    """Gated DeltaNet with FP8 inputs (E4M3 q, k, v with per-row scales, decoded
    on chip; fp32 state, bf16 output) on the runner's tree: the row quantisation
    runs once outside the timed launches (HIP events on the launch stream,
    eager). Algorithmic bytes: those of the bf16 layer with 1-byte q, k, v and
    three fp32 scales per (token, head). Returns the timing and the output
    (for the fidelity check)."""
    import torch

    t = r.t
    T, gH, dk, dv = meta["T"], meta["gH"], meta["dk"], meta["dv"]
    q8, qs = r.sess.quantize_fp8(t["gq"][:T].reshape(T * gH, dk))
    k8, ks = r.sess.quantize_fp8(t["gk"][:T].reshape(T * gH, dk))
    v8, vs = r.sess.quantize_fp8(t["gv"][:T].reshape(T * gH, dv))
    go = torch.empty((T, gH, dv), dtype=torch.bfloat16, device="cuda")
    r.build()
    run = lambda: r.sess.gdn_fp8(q8.view(T, gH, dk), qs.view(T, gH), k8.view(T, gH, dk), ks.view(T, gH),
                                 v8.view(T, gH, dv), vs.view(T, gH), t["a"], t["b"], go, r.st0,
                                 root_state=t.get("root_state"))
    for _ in range(warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    st = stats_us([e0.elapsed_time(e1) for e0, e1 in evs])
    parent, seg_len = meta["parent"], meta["seg_len"]
    gb = gdn_work(parent, seg_len, gH, dk, dv, 2, meta.get("root_state", False))
    gb -= T * gH * (2 * dk + dv) * 1.0  # q, k, v: 1 byte per element instead of 2
    gb += T * gH * 12.0                  # their three row scales
    return dict(p50_us=st["p50_us"], p95_us=st["p95_us"], mean_us=st["mean_us"],
                achieved_gbs=gb / (st["mean_us"] * 1e-6) / 1e9, hbm_frac=gb / PEAK_HBM / (st["mean_us"] * 1e-6),
                algorithmic_bytes=gb,
                note="gdn_fork_forward_fp8, eager, every segment on gdn_fused_kernel<128, true>; fidelity against "
                     "the float32 oracle on the unquantised inputs is in fidelity.gdn_fp8_inputs", o=go)


def host_threads() -> int:
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------------- workloads

def build_workload(name, threads=8):
    """(meta dict, device tensors, host workload or None) of a named workload;
    every input is the seeded PCG64 draw of the workloads module."""
    from tree_structured_decision_amd import workloads as W
    from tree_structured_decision_amd.session import request_mix_to_device

    if name in ("tiny_one_level", "one_request", "wide_options", "agent_history"):
        wl = W.WORKLOADS[name]()
        meta = wl_meta_of(wl.parent, wl.seg_len, wl.H, wl.Hkv, wl.D, wl.gH, wl.dk, wl.dv, wl.dtype)
        meta["root_state"] = wl.root_state is not None
        return meta, tensors_from_numpy(wl), wl
    if name == "agent_history_resume":
        # the agent-history request resumed from a checkpoint of its 4096-token
        # root: that prefix's keys/values come from the cache (shared by the 8
        # children, now roots of the stream) and its recurrent state is the
        # children's root state; the stream holds the 8 x 512 children and the
        # options only
        wl = W.agent_history()
        P = int(wl.seg_len[0])
        parent = (wl.parent[1:] - (wl.parent[1:] >= 0)).astype(np.int32)
        seg_len = wl.seg_len[1:].astype(np.int32)
        roots = parent < 0
        meta = wl_meta_of(parent, seg_len, wl.H, wl.Hkv, wl.D, wl.gH, wl.dk, wl.dv, wl.dtype)
        meta["ctx"] = (np.zeros(len(parent), np.int32), np.where(roots, P, 0).astype(np.int32), P)
        meta["root_state"] = True
        full = tensors_from_numpy(wl)
        t = {n: full[n][P:].contiguous() for n in ("q", "k", "v", "gq", "gk", "gv", "a", "b")}
        t["kc"], t["vc"] = full["k"][:P].contiguous(), full["v"][:P].contiguous()
        t["root_state"] = full["root_state"].expand(int(roots.sum()), -1, -1, -1).contiguous()
        return meta, t, None
    if name == "request_mix":
        from tree_structured_decision_amd.session import pick_bucket

        rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 5))
        p0, l0 = W.request_mix_tree(rng)
        t_cap, _ = pick_bucket(int(l0.sum()), len(p0))  # drawn straight into the bucket's rows
        parent, seg_len, t, w = request_mix_to_device(W.SEED_BASE + 5, t_cap, threads=threads)
        meta = wl_meta_of(parent, seg_len, 16, 2, 128, 16, 128, 128)
        meta["root_state"] = False
        meta["readout"] = w
        return meta, t, None
    raise ValueError(name)


def layer_fracs(meta, res):
    """Per-layer roofline fractions of an eager timing (P50 and mean)."""
    elt = 2 if meta["dtype"] == "bf16" else 4
    ctx = meta.get("ctx")
    fl, ab = attn_work(meta["parent"], meta["seg_len"], meta["H"], meta["Hkv"], meta["D"], elt,
                       ctx_len=None if ctx is None else ctx[1], ctx_rows=0 if ctx is None else ctx[2])
    gb = gdn_work(meta["parent"], meta["seg_len"], meta["gH"], meta["dk"], meta["dv"], elt,
                  meta.get("root_state", False))
    peak = PEAK_BF16_MFMA if meta["dtype"] == "bf16" else PEAK_F32_MFMA
    a_roof = max(fl / peak, ab / PEAK_HBM)
    g_roof = gb / PEAK_HBM
    return dict(attn_flop=fl, attn_bytes=ab, gdn_bytes=gb, attn_roof_s=a_roof, gdn_roof_s=g_roof,
                attn_bound="mfma" if fl / peak >= ab / PEAK_HBM else "hbm", peak_mfma=peak)


def workload_report(meta, eager, graph):
    f = layer_fracs(meta, eager)
    T = meta["T"]
    a, g = eager["attention"], eager["gdn"]
    rep = dict(tokens=T, segments=meta["S"],
               eager=dict(stream_tokens_per_s=T / (eager["ms_per_step"] * 1e-3),
                          ms_per_step=eager["ms_per_step"],
                          pair_p50_us=eager["pair"]["p50_us"], pair_p95_us=eager["pair"]["p95_us"],
                          attn_p50_us=a["p50_us"], attn_p95_us=a["p95_us"],
                          gdn_p50_us=g["p50_us"], gdn_p95_us=g["p95_us"]),
               attn_tflops=f["attn_flop"] / (a["p50_us"] * 1e-6) / 1e12,
               attn_frac=f["attn_roof_s"] / (a["p50_us"] * 1e-6), attn_bound=f["attn_bound"],
               gdn_gbs=f["gdn_bytes"] / (g["p50_us"] * 1e-6) / 1e9,
               gdn_hbm_frac=f["gdn_roof_s"] / (g["p50_us"] * 1e-6),
               pair_roofline_frac=(f["attn_roof_s"] + f["gdn_roof_s"]) / (eager["pair"]["p50_us"] * 1e-6))
    if graph is not None:
        rep["graph"] = dict(stream_tokens_per_s=T / (graph["ms_per_step"] * 1e-3),
                            ms_per_step=graph["ms_per_step"], pair_p50_us=graph["pair"]["p50_us"],
                            pair_p95_us=graph["pair"]["p95_us"],
                            pair_roofline_frac=(f["attn_roof_s"] + f["gdn_roof_s"]) /
                            (graph["pair"]["p50_us"] * 1e-6))
    return rep


def run_workload(name, steps, warmup, threads):
    """Eager and graph-replay timings of one workload (both in one capacity-
    bucket session: eager launches are sized from the host plan)."""
    import torch

    meta, t, _ = build_workload(name, threads)
    r = Runner(meta, t, graph=True)
    eager = time_runner(r, steps, warmup, eager=True)
    graph = time_runner(r, steps, warmup, eager=False)
    rep = workload_report(meta, eager, graph)
    r.close()
    del r, t
    torch.cuda.empty_cache()
    return rep


def all_workloads(steps, warmup, threads):
    rep = {}
    for name in ("tiny_one_level", "one_request", "wide_options", "agent_history", "agent_history_resume"):
        log(f"workload {name}")
        rep[name] = run_workload(name, steps, warmup, threads)
        log(f"  {json.dumps(rep[name])}")
    return rep


# --------------------------------------------------------------- CPU baseline

def request_cost(parent, seg_len):
    """Relative oracle work of one request: the Gated DeltaNet recurrence runs
    every segment's whole path (path tokens), attention its visible pairs."""
    parent = np.asarray(parent)
    seg_len = np.asarray(seg_len, np.int64)
    path = np.zeros(len(parent), np.int64)
    for s in range(len(parent)):
        path[s] = seg_len[s] + (path[parent[s]] if parent[s] >= 0 else 0)
    return float(path.sum()) * 6 * 128 * 128 + 2.0 * 128 * visible_pairs(parent, seg_len)


def cpu_baseline_mix(meta, o_gpu_rows, go_gpu_rows, threads, o8_rows=None, go8_rows=None):
    """The float32 oracle (both layers) on a prefix of the request mix's
    requests, in stream order, about CPU_BUDGET_S seconds of work on `threads`
    cores: the first request calibrates the cost per work unit, and the
    prefix stops before the request that would overrun the budget. Returns
    (cpu_baseline entry, fidelity of those requests' option softmax scores
    against the oracle). o_gpu_rows(t0, t1) / go_gpu_rows(t0, t1): the GPU
    outputs of stream rows [t0, t1) as float64 arrays (o8_rows / go8_rows: those
    of the FP8 variants, or None)."""
    import oracle
    from tree_structured_decision_amd import metrics
    from tree_structured_decision_amd import workloads as W

    oracle.set_threads(threads, "f32")
    parent, seg_len = meta["parent"], meta["seg_len"]
    spans = W.request_spans(parent, seg_len)
    w = meta["readout"]
    used, tokens, took, rate = [], 0, 0.0, None
    fid_a, fid_g, fid_8, fid_g8 = [], [], [], []
    for r, (a, b, t0, t1) in enumerate(spans):
        cost = request_cost(np.where(parent[a:b] >= 0, parent[a:b] - a, -1), seg_len[a:b])
        if rate is not None and took + cost / rate > CPU_BUDGET_S:
            break
        wl = W.request_mix_request(W.SEED_BASE + 5, r, parent, seg_len, w=w)
        tic = time.perf_counter()
        o, _ = oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, prec="f32")
        go, _, _ = oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b, prec="f32")
        dt = time.perf_counter() - tic
        took += dt
        if rate is None:
            rate = cost / dt  # work units per second, from the first request
        tokens += wl.T
        used.append(r)
        fid_a.append(metrics.decision_fidelity(o_gpu_rows(t0, t1), o, wl.w_attn, wl.parent, wl.seg_len))
        fid_g.append(metrics.decision_fidelity(go_gpu_rows(t0, t1), go, wl.w_gdn, wl.parent, wl.seg_len))
        if o8_rows is not None:
            fid_8.append(metrics.decision_fidelity(o8_rows(t0, t1), o, wl.w_attn, wl.parent, wl.seg_len))
        if go8_rows is not None:
            fid_g8.append(metrics.decision_fidelity(go8_rows(t0, t1), go, wl.w_gdn, wl.parent, wl.seg_len))
    agg = lambda fs: dict(groups=len(fs), tvd_max=max(f["tvd_max"] for f in fs),
                          tvd_mean=float(np.mean([f["tvd_mean"] for f in fs])),
                          argmax_agreement=float(np.mean([f["argmax_agreement"] for f in fs])))
    cpu = dict(value=tokens / took, unit="tokens/s", cores=threads, kind="oracle",
               sample=f"requests 0..{used[-1]} of the request mix ({len(used)} of {len(spans)} requests, "
                      f"{tokens} of {meta['T']} stream tokens; both layers, float32 oracle, "
                      f"{took:.1f} s wall on {threads} threads)",
               cpu_model=cpu_model(), host_cores=os.cpu_count())
    fid = dict(attention=agg(fid_a), gdn=agg(fid_g), attention_fp8_scores=agg(fid_8) if fid_8 else None,
               gdn_fp8_inputs=agg(fid_g8) if fid_g8 else None,
               reference=f"float32 oracle, the {len(used)} requests of the CPU-baseline sample, one "
                         "decision group per request")
    return cpu, fid


def cpu_stack_fidelity(wl, stack_inputs):
    """The float32 oracle of the hybrid stack (unrounded intermediates) as the
    reference of the option distributions' total-variation distance."""
    import oracle
    from oracle import mixer as OM
    from tree_structured_decision_amd import metrics

    h_gpu, h8_gpu, x0, layers, fn, w_head = stack_inputs
    t0 = time.perf_counter()
    ref = OM.stack(wl.parent, wl.seg_len, x0, layers, fn, prec="f32")
    fid = metrics.decision_fidelity(h_gpu, ref, w_head, wl.parent, wl.seg_len)
    fid["reference"] = "float32 oracle (unrounded intermediates)"
    fid["oracle_s"] = time.perf_counter() - t0
    fid8 = metrics.decision_fidelity(h8_gpu, ref, w_head, wl.parent, wl.seg_len)
    fid8["reference"] = "float32 oracle without quantisation (the cost of FP8 projections)"
    return fid, fid8



def readout_entry(r: "Runner", meta, iters=50):
    """The decision readout on the GPU (fork_option_readout) over the attention
    output the last step left in r.o: per-option scores and per-group softmax
    probabilities of every decision group of the tree. Event-timed over
    `iters` calls; compared with the host float64 readout of the same rows."""
    import torch
    from tree_structured_decision_amd import metrics

    parent = np.asarray(meta["parent"])
    seg_len = np.asarray(meta["seg_len"], np.int64)
    C = r.o[0].numel()
    w = torch.from_numpy(np.random.default_rng(7).standard_normal(C).astype(np.float32)).cuda()
    score, prob = r.sess.option_readout(r.o, w)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        r.sess.option_readout(r.o, w, score, prob)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    last = torch.from_numpy(np.cumsum(seg_len) - 1).cuda()
    rows = r.o.index_select(0, last).float().cpu().numpy().astype(np.float64)
    host = metrics.option_scores(rows, w.cpu().numpy(), parent, np.ones_like(seg_len))
    p_gpu = prob.cpu().numpy().astype(np.float64)
    err = max(float(np.abs(p_gpu[list(leaves)] - metrics.softmax64(sc)).max()) for leaves, sc in host.values())
    n_opt = sum(len(leaves) for leaves, _ in host.values())
    return dict(us=us, options=n_opt, groups=len(host), row_values=C,
                max_abs_prob_diff_vs_host_fp64=err,
                note="fork_option_readout on the attention output [T, 16 x 128] bf16: score = <w, last row> "
                     "/ sqrt(C) per option, softmax per decision group (leaves sharing a parent); two "
                     "launches, HIP events over the calls")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-workloads", action="store_true", help="headline workload only")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the block-piece, mixer and stack legs (kernel profiles of the step)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak pass")
    ap.add_argument("--only", default=None,
                    help="time just this workload, eager and graph replay (profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="finish with three plain 512 MiB device copies (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the hot path runs on one GPU (got --gpus {args.gpus}); "
              "sharding across GPUs is described in the design notes, not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    log(f"device: {torch.cuda.get_device_name(0)}")
    threads = host_threads()

    if args.only:
        print(json.dumps({args.only: run_workload(args.only, args.steps, args.warmup, threads)}), flush=True)
        calib_copy(args.calib_copy)
        return

    # ---------------- headline: the request mix, graph replay of its bucket
    meta, t, _ = build_workload("request_mix", threads)
    T, S = meta["T"], meta["S"]
    r = Runner(meta, t, graph=True)
    log(f"headline request_mix: T={T} S={S}, bucket {r.caps}; warmup {args.warmup}, steps {args.steps}")
    graph = time_runner(r, args.steps, args.warmup, eager=False)
    eager = time_runner(r, args.steps, args.warmup, eager=True)
    fp8 = fp8_scores(r, meta, args.steps, args.warmup)
    gdn8 = fp8_gdn(r, meta, args.steps, args.warmup)
    r.step()  # leave the graph replay's outputs in place for the fidelity check
    torch.cuda.synchronize()
    readout = readout_entry(r, meta)
    f = layer_fracs(meta, eager)
    a_mean = eager["attention"]["mean_us"] * 1e-6
    g_mean = eager["gdn"]["mean_us"] * 1e-6
    attn_ach = f["attn_flop"] / a_mean
    gdn_ach = f["gdn_bytes"] / g_mean
    tr_a = measured_traffic("fork_attn_forward", "request_mix")
    tr_g = measured_traffic("gdn_fork_forward", "request_mix")
    roof = dict(bound="mfma", achieved=attn_ach / 1e12, peak=PEAK_BF16_MFMA / 1e12, unit="TFLOP/s",
                frac=attn_ach / PEAK_BF16_MFMA, traffic=None if tr_a is None else tr_a["bytes"],
                kernel="fork_attn_kernel (fork_attn_forward)",
                algorithmic_per_launch=f["attn_flop"], launch_mean_us=a_mean * 1e6,
                algorithmic_bytes=f["attn_bytes"],
                note="4 D H flops per visible (query, key) pair, 1 launch per step (no split tiles on "
                     "this tree, so no merge launch); mean duration over the timed steps, HIP events on "
                     "the launch stream (eager launch of the same tree in the same bucket session); "
                     "kernel trace in profiles/request_mix_kernels.md")
    roof_g = dict(bound="hbm", achieved=gdn_ach / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s",
                  frac=gdn_ach / PEAK_HBM, traffic=None if tr_g is None else tr_g["bytes"],
                  kernel="gdn_fork_forward (gdn_prep_kernel + per-depth scans)",
                  algorithmic_per_launch=f["gdn_bytes"], launch_mean_us=g_mean * 1e6,
                  note="q, k, v, o, a, b of the stream and S - R fork copies of the fp32 state")

    cpu = fid = None
    if not args.no_cpu:
        log(f"cpu baseline: float32 oracle on a prefix of the requests, {threads} threads")
        ho = lambda x: (lambda t0, t1: x[t0:t1].float().cpu().numpy().astype(np.float64))
        cpu, fid = cpu_baseline_mix(meta, ho(r.o), ho(r.go), threads, o8_rows=ho(fp8.pop("o")),
                                    go8_rows=ho(gdn8.pop("o")))
    else:
        fp8.pop("o")
        gdn8.pop("o")
    n_opt, opt_tok, iso_tok = tree_rates(meta["parent"], meta["seg_len"])
    step_s = graph["ms_per_step"] * 1e-3
    rates = dict(options=n_opt, option_tokens_per_s=opt_tok / step_s,
                 isolated_equivalent_tokens_per_s=iso_tok / step_s, us_per_option=step_s / n_opt * 1e6,
                 note="per graph step (wall); isolated-equivalent = sum over options of the root-to-option "
                      "path length")
    layers = dict(graph_pair=graph["pair"], eager_attention=eager["attention"], eager_gdn=eager["gdn"],
                  eager_pair=eager["pair"], eager_ms_per_step=eager["ms_per_step"],
                  eager_stream_tokens_per_s=T / (eager["ms_per_step"] * 1e-3))
    r.close()
    del r, t
    torch.cuda.empty_cache()

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        roof["frac_measured_peak"] = roof["achieved"] / peaks["bf16_gemm_tflops"]
        roof_g["frac_measured_peak"] = roof_g["achieved"] / peaks["copy_gbs"]
    out = {
        "metric": METRIC,
        "value": T / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": graph["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "request_mix: 64 decision requests in one stream (prefix 1/P on 256..16384, "
                               "options 1/n on 2..256 of U{4..32} tokens), bf16, attention 16 q / 2 kv heads "
                               "x 128, Gated DeltaNet 16 x 128 x 128; graph replay of the 393216-token x "
                               "4096-segment bucket; seeded PCG64 inputs (seed 1005)",
                   "tokens": T, "segments": S, "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_gdn": roof_g,
        "cpu_baseline": cpu,
        "fidelity": fid,
        "layers": layers,
        "attention_fp8_scores": fp8,
        "gdn_fp8_inputs": gdn8,
        "rates": rates,
        "readout": readout,
        "measured_peaks": peaks,
    }
    if not args.no_workloads:
        out["workloads"] = all_workloads(max(5, args.steps // 2), 3, threads)
    if not args.no_extras:
        from tree_structured_decision_amd import workloads as W
        from tree_structured_decision_amd.session import ForkSession, caps_for

        wl = W.one_request()
        caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv)
        sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
        sess.build(wl.parent, wl.seg_len)
        out["block_ops"] = {"one_request": block_ops(wl, sess)}
        out["mixers"] = {"one_request": mixer_ops(wl, sess)}
        st, st_inputs = stack_ops(wl, sess)
        if not args.no_cpu:
            st["fidelity"], st["fp8_fidelity"] = cpu_stack_fidelity(wl, st_inputs)
        out["stack"] = {"one_request": st}
        sess.close()
    print(json.dumps(out), flush=True)
    calib_copy(args.calib_copy)


def block_ops(wl, sess, iters=50):
    """The fork-aware block pieces on a workload's tree (metadata already built in
    sess): rotary embedding of the attention q and k heads, and the short
    convolution of the Gated DeltaNet q | k | v channels (width 4, SiLU). Each
    is HBM-bound: algorithmic bytes = one read and one write of the
    activations; timed with HIP events on the launch stream."""
    import torch

    bf = torch.bfloat16
    T = wl.T
    q = torch.randn(T, wl.H, wl.D, device="cuda").to(bf)
    k = torch.randn(T, wl.Hkv, wl.D, device="cuda").to(bf)
    C = 3 * wl.gH * wl.dk
    x = torch.randn(T, C, device="cuda").to(bf)
    y = torch.empty_like(x)
    w = torch.randn(C, 4, device="cuda") * 0.5
    ops = {
        "rope_q_k": (lambda: (sess.rope(q), sess.rope(k)), 2.0 * (q.numel() + k.numel()) * 2),
        "conv_qkv": (lambda: sess.conv(x, w, y, act=1), 2.0 * x.numel() * 2 + w.numel() * 4),
    }
    rep = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / iters
        rep[name] = dict(us=t * 1e6, algorithmic_bytes=nbytes, achieved_gbs=nbytes / t / 1e9,
                         hbm_frac=nbytes / t / PEAK_HBM)
    rep["note"] = ("fork_rope_forward on q [T,16,128] and k [T,2,128]; fork_conv_forward on "
                   f"[T,{C}] (q | k | v of the Gated DeltaNet), width 4, SiLU; bf16")
    return rep


def mixer_ops(wl, sess, iters=20, dm=2048):
    """Both token mixers of a hybrid block of model width dm on a workload's tree
    (metadata already built in sess), random bf16 weights: the attention mixer
    (q, k, v, gate projections, rotary embedding, tree attention, sigmoid gate,
    output projection) and the Gated DeltaNet mixer (q | k | v, decay / strength
    and output-gate projections, convolution, normalised inputs, forked Gated
    DeltaNet, gated RMS norm, output projection). Timed with HIP events on the
    launch stream; the projections alone are timed too, as plain GEMMs against
    the bf16 MFMA peak, and the per-token kernels against HBM."""
    import torch

    from tree_structured_decision_amd import workloads as W

    T = wl.T
    Wt = W.mixer_weights(SEED_MIXER, dm, H=wl.H, Hkv=wl.Hkv, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
    dev = lambda a, dt=torch.bfloat16: torch.from_numpy(a).to("cuda", dt)
    A = sess.fuse_attention_weights({n: (dev(v) if isinstance(v, np.ndarray) else v)
                                     for n, v in Wt["attn"].items()})
    G = sess.fuse_gdn_weights({n: (dev(v) if isinstance(v, np.ndarray) and n.startswith("w") else
                                   dev(v, torch.float32) if isinstance(v, np.ndarray) else v)
                               for n, v in Wt["gdn"].items()})
    x = dev(W.mixer_input(SEED_MIXER + 1, T, dm))
    ab, gb = {}, {}
    C = 2 * wl.gH * wl.dk + wl.gH * wl.dv
    proj = [(A["wqkvg"], "f"), (G["wqkv"], "p"), (G["wzab"], "zab")]
    outs = {}

    def projections():
        for w, n in proj:
            if n not in outs:
                outs[n] = torch.empty(T, w.shape[0], dtype=torch.bfloat16, device="cuda")
            sess.linear(x, w, outs[n])
        if "u" not in outs:
            outs["u"] = torch.randn(T, wl.H * wl.D, device="cuda").to(torch.bfloat16)
            outs["ug"] = torch.randn(T, wl.gH * wl.dv, device="cuda").to(torch.bfloat16)
            outs["y"] = torch.empty(T, dm, dtype=torch.bfloat16, device="cuda")
        sess.linear(outs["u"], A["wo"], outs["y"])
        sess.linear(outs["ug"], G["wo"], outs["y"])

    flop = 2.0 * T * dm * (sum(w.shape[0] for w, _ in proj) + wl.H * wl.D + wl.gH * wl.dv)  # + 2 outputs
    o = torch.randn(T, wl.H, wl.D, device="cuda").to(torch.bfloat16)
    g = torch.randn_like(o)
    og = torch.randn(T, wl.gH, wl.dv, device="cuda").to(torch.bfloat16)
    zg = torch.randn_like(og)
    u = torch.empty_like(o)
    ug = torch.empty_like(og)
    c = torch.randn(T, C, device="cuda").to(torch.bfloat16)
    abp = torch.randn(T, 2 * wl.gH, device="cuda").to(torch.bfloat16)
    q = torch.empty(T, wl.gH, wl.dk, dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty(T, wl.gH, wl.dv, dtype=torch.bfloat16, device="cuda")
    aa = torch.empty(T, wl.gH, device="cuda")
    bb = torch.empty_like(aa)
    # FP8: weights quantised per output channel once; activations per token inside
    A8, G8 = sess.quantize_weights(A), sess.quantize_weights(G)
    ab8, gb8, outs8 = {}, {}, {}
    xq, xs = sess.quantize_fp8(x)
    proj8 = [(A8["wqkvg"], "f"), (G8["wqkv"], "p"), (G8["wzab"], "zab")]

    def projections_fp8():
        for (wq_, ws_), n in proj8:
            if n not in outs8:
                outs8[n] = torch.empty(T, wq_.shape[0], dtype=torch.bfloat16, device="cuda")
            sess.linear_fp8(xq, xs, wq_, ws_, outs8[n])
        if "u" not in outs8:
            outs8["u"] = sess.quantize_fp8(torch.randn(T, wl.H * wl.D, device="cuda").to(torch.bfloat16))
            outs8["ug"] = sess.quantize_fp8(torch.randn(T, wl.gH * wl.dv, device="cuda").to(torch.bfloat16))
            outs8["y"] = torch.empty(T, dm, dtype=torch.bfloat16, device="cuda")
        sess.linear_fp8(*outs8["u"], *A8["wo"], outs8["y"])
        sess.linear_fp8(*outs8["ug"], *G8["wo"], outs8["y"])

    xq_buf = torch.empty(T, dm, dtype=torch.uint8, device="cuda")
    xs_buf = torch.empty(T, device="cuda")
    ops = {
        "attention_mixer": (lambda: sess.attention_mixer(x, A, bufs=ab), None, None),
        "attention_mixer_fp8": (lambda: sess.attention_mixer(x, A8, bufs=ab8, fp8=True), None, None),
        "gdn_mixer_fp8": (lambda: sess.gdn_mixer(x, G8, bufs=gb8, fp8=True), None, None),
        "projections_fp8": (projections_fp8, "mfma8", flop),
        "quantize_fp8": (lambda: sess.quantize_fp8(x, xq_buf, xs_buf), "hbm", x.numel() * 3.0 + T * 4),
        "gdn_mixer": (lambda: sess.gdn_mixer(x, G, bufs=gb), None, None),
        "projections": (projections, "mfma", flop),
        "gate_sigmoid": (lambda: sess.gate(o, g, None, u, 0), "hbm", 3.0 * o.numel() * 2),
        "gated_rmsnorm": (lambda: sess.gate(og, zg, G["norm_w"], ug, 1), "hbm", 3.0 * og.numel() * 2),
        "gdn_inputs": (lambda: sess.gdn_inputs(c, abp, G["a_log"], G["dt_bias"], q, k, v, aa, bb), "hbm",
                       2.0 * c.numel() * 2 + abp.numel() * 2 + 2 * aa.numel() * 4),
    }
    rep = {}
    for name, (fn, bound, work) in ops.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / iters
        r = dict(us=t * 1e6)
        if bound == "mfma":
            r.update(algorithmic_flop=work, achieved_tflops=work / t / 1e12, mfma_frac=work / t / PEAK_BF16_MFMA)
        elif bound == "mfma8":
            r.update(algorithmic_flop=work, achieved_tflops=work / t / 1e12, mfma_frac=work / t / PEAK_FP8_MFMA)
        elif bound == "hbm":
            r.update(algorithmic_bytes=work, achieved_gbs=work / t / 1e9, hbm_frac=work / t / PEAK_HBM)
        rep[name] = r
    pair = rep["attention_mixer"]["us"] + rep["gdn_mixer"]["us"]
    rep["mixer_pair_us"] = pair
    rep["mixer_pair_tokens_per_s"] = T / (pair * 1e-6)
    pair8 = rep["attention_mixer_fp8"]["us"] + rep["gdn_mixer_fp8"]["us"]
    rep["mixer_pair_fp8_us"] = pair8
    rep["mixer_pair_fp8_tokens_per_s"] = T / (pair8 * 1e-6)
    rep["note"] = (f"model width {dm}; attention 16 q / 2 kv heads x 128, Gated DeltaNet 16 heads x 128, "
                   "convolution width 4; random bf16 weights; projections = the 5 GEMMs of both "
                   "mixers (hipBLASLt, fp32 accumulation; the attention mixer's q | k | v | gate "
                   "projections run as one product whose output is split into heads by the rotary "
                   "kernel, the Gated DeltaNet's output gate and decay / strength projections as "
                   "another); *_fp8: E4M3 projections with per-token "
                   "activation and per-channel weight scales (quantisation inside the mixers, "
                   "against the fp8 MFMA peak)")
    return rep


def stack_ops(wl, sess, iters=10, dm=2048):
    """A four-layer hybrid stack (Gated DeltaNet, attention, Gated DeltaNet,
    attention; pre-norm residual, model width dm, random bf16 weights) on a
    workload's tree, then the option readout: per decision group, the softmax
    of <w_head, h at each option's last token>. Reports the time per stack pass
    (HIP events on the launch stream) and the total-variation distance of the
    option distributions to the float32 oracle's (the fidelity measure of the
    pages, computed in the CPU-baseline leg), with argmax agreement. Returns the
    report and what that leg needs (the GPU's final hidden states, the inputs
    and weights)."""
    import torch

    from tree_structured_decision_amd import workloads as W

    T = wl.T
    layers, fn, w_head = W.stack_weights(SEED_MIXER + 10, dm, H=wl.H, Hkv=wl.Hkv, D=wl.D, gH=wl.gH,
                                         dk=wl.dk, dv=wl.dv)

    def dev(a, bf=False):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
            "cuda", torch.bfloat16 if bf else torch.float32)

    dl = []
    for k, Wl, nw in layers:
        Wd = {n: (dev(v, n.startswith("w") and v.ndim == 2) if isinstance(v, np.ndarray) else v)
              for n, v in Wl.items()}
        dl.append((k, sess.fuse_attention_weights(Wd) if k == "attn" else sess.fuse_gdn_weights(Wd), dev(nw)))
    dfn = dev(fn)
    x0 = W.mixer_input(SEED_MIXER + 20, T, dm)
    x0d = dev(x0, True)
    x = torch.empty_like(x0d)
    dl8 = [(k, sess.quantize_weights(Wl), nw) for k, Wl, nw in dl]

    def timed(fp8):
        bufs = {}

        def once():
            x.copy_(x0d)
            return sess.stack(x, dl8 if fp8 else dl, dfn, bufs=bufs, fp8=fp8)

        for _ in range(2):
            once()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            h = once()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / iters, h.float().cpu().numpy().astype(np.float64)

    t, h_gpu = timed(False)
    t8, h8_gpu = timed(True)
    rep = dict(layers=[k for k, _, _ in layers], model_width=dm, us=t * 1e6, tokens_per_s=T / t,
               fp8_us=t8 * 1e6, fp8_tokens_per_s=T / t8, fidelity=None, fp8_fidelity=None)
    rep["note"] = ("pre-norm residual stack; the residual add happens in the output projections; "
                   "each pass includes a copy of the input into the residual stream")
    return rep, (h_gpu, h8_gpu, x0, layers, fn, w_head)


def calib_copy(enabled: bool):
    """Three copies of 512 MiB (the known-size kernel HBM counters are scaled by)."""
    if not enabled:
        return
    import torch

    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration: 3 device copies of {n >> 20} MiB")




if __name__ == "__main__":
    main()
