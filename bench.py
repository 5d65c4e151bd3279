"""Benchmark of the ForkAttention hot path on one MI355X.

A step is one pass of the whole path over one decision request: segment
metadata build (host plan + upload + per-token expansion), tree attention and
the forked Gated DeltaNet layer. The headline workload is one decision request
(prefix 2048 + 16 options of 16-48 tokens, bf16, attention 16/2/128, Gated
DeltaNet 16 x 128 x 128). `value` is stream tokens per second (every physical
token counted once) with inputs resident in HBM.

Also reported on the same JSON line:
  roofline      the dominant kernel's algorithmic work per launch over its mean
                launch time (HIP events on the launch stream) vs MI355X peak;
  cpu_baseline  the CPU oracle timed on this host's cores on the same request;
  fidelity      total-variation distance of per-option softmax scores vs the
                float32 oracle, argmax agreement;
  workloads     throughput of all five synthetic workloads (the request mix
                runs as graph replay of a capacity bucket);
  rates         option tokens/s, isolated-equivalent tokens/s, us per option;
  cold_cache    the layer pair's kernel times with caches evicted between steps;
  measured_peaks  a bf16 GEMM and a device copy on this GPU, the achievable
                peaks the roofline fraction is also given against;
  block_ops     the fork-aware rotary embedding and short convolution;
  mixers        both token mixers of a hybrid block (model width 2048): the
                projections against the MFMA peak, the per-token kernels
                against HBM;
  stack         a four-layer hybrid stack and the option distributions' TVD
                to the float32 oracle (computed in the CPU-baseline leg).
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


def measured_traffic(kernel: str):
    """HBM bytes per call of `kernel` from the committed counter runs
    (profiles/hbm_traffic.json), or None when any native source has changed
    since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256():
        return None
    return dict(bytes=rec["read_bytes"] + rec["write_bytes"], read=rec["read_bytes"],
                write=rec["write_bytes"], workload=rec["workload"], summary=rec["summary"])


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
    """Algorithmic flops (visible pairs) and bytes (q, k, v, o of the stream,
    plus the cached context's k, v read once)."""
    T = int(np.sum(seg_len))
    flops = 4.0 * D * H * visible_pairs(parent, seg_len, ctx_len)
    bytes_ = float(T * (2 * H + 2 * Hkv) * D * elt + ctx_rows * 2 * Hkv * D * elt)
    return flops, bytes_


def gdn_work(parent, seg_len, H, dk, dv, elt, root_state: bool):
    T = int(np.sum(seg_len))
    S = len(parent)
    R = int(np.sum(np.asarray(parent) < 0))
    io = T * H * ((2 * dk + 2 * dv) * elt + 8)        # q, k, v, o + a, b
    fork = S * H * dk * dv * 4                         # every segment's start state written once
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

class Runner:
    """Device buffers and one step of the path for one workload."""

    def __init__(self, wl_meta: dict, tensors: dict, graph: bool):
        import torch
        from tree_structured_decision_amd.session import ForkSession

        self.m = wl_meta
        self.t = tensors
        T, S = wl_meta["T"], wl_meta["S"]
        depth = wl_meta["depth"]
        if graph:
            from tree_structured_decision_amd.session import BUCKET_DEPTH, pick_bucket

            t_cap, s_cap = pick_bucket(T, S)
            depth_cap = max(BUCKET_DEPTH, depth)
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
        self.o = torch.empty((t_cap, H, D), dtype=qd, device=dev)
        self.lse = torch.empty((t_cap, H), dtype=torch.float32, device=dev)
        self.go = torch.empty((t_cap, gH, dv), dtype=qd, device=dev)
        self.st0 = torch.empty((s_cap, gH, dv, dk), dtype=torch.float32, device=dev)
        self.graph = graph
        self._build()
        if graph:
            t = tensors
            self.sess.capture(dict(q=t["q"], k=t["k"], v=t["v"], o=self.o, lse=self.lse),
                              dict(q=t["gq"], k=t["gk"], v=t["gv"], a=t["a"], b=t["b"],
                                   root_state=t.get("root_state"), o=self.go,
                                   seg_start_state=self.st0))

    def _build(self):
        if self.ctx is None:
            self.sess.build(self.m["parent"], self.m["seg_len"])
        else:
            self.sess.build(self.m["parent"], self.m["seg_len"], ctx_start=self.ctx[0],
                            ctx_len=self.ctx[1])

    def step(self, ev=None):
        t = self.t
        self._build()
        if self.graph:
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


def time_runner(r: Runner, steps: int, warmup: int, evict=None):
    """Times `steps` steps after `warmup`, twice: first the plain steps between
    two synchronisations (the wall time per step: nothing else is enqueued),
    then the same number of steps with HIP events around each layer (per-layer
    durations; an event record costs a few microseconds of GPU time, so this
    pass is not the one the wall time comes from). evict: a large device buffer
    written before every step of the event pass (outside the events), so that
    the step's inputs come from HBM rather than the L2 / Infinity Cache; then
    the wall pass is skipped."""
    import torch

    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    wall = None
    if evict is None:
        t0 = time.perf_counter()
        for _ in range(steps):
            r.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        if evict is not None:
            evict.fill_(k & 0xff)
        r.step(evs[k])
    torch.cuda.synchronize()
    if wall is None:
        wall = time.perf_counter() - t0
    if r.graph:
        pair = [e[0].elapsed_time(e[2]) for e in evs]
        attn = gdn = None
    else:
        attn = [e[0].elapsed_time(e[1]) for e in evs]
        gdn = [e[1].elapsed_time(e[2]) for e in evs]
        pair = [a + g for a, g in zip(attn, gdn)]
    med = lambda x: None if x is None else float(np.median(x)) * 1e-3  # seconds
    mean = lambda x: None if x is None else float(np.mean(x)) * 1e-3
    return dict(wall=wall, ms_per_step=wall / steps * 1e3, attn_mean=mean(attn),
                attn_p50=med(attn), gdn_mean=mean(gdn), gdn_p50=med(gdn), pair_p50=med(pair),
                pair_p95=None if pair is None else float(np.percentile(pair, 95)) * 1e-3)


def tensors_from_numpy(wl):
    from tree_structured_decision_amd.session import to_device

    return to_device(wl, "cuda")


def tensors_on_device(name, parent, seg_len, H, Hkv, D, gH, dk, dv, seed, gates, root_std):
    """Draw a workload's tensors directly on the GPU (same shapes and
    distributions as the numpy workloads; used for the large ones where a
    host-side draw would dominate the run)."""
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    T = int(np.sum(seg_len))
    R = int(np.sum(np.asarray(parent) < 0))
    bf = torch.bfloat16
    rn = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32)
    q = rn(T, H, D).to(bf)
    k = rn(T, Hkv, D).to(bf)
    v = rn(T, Hkv, D).to(bf)
    gq = rn(T, gH, dk).to(bf)
    gk = rn(T, gH, dk)
    gk = (gk / gk.norm(dim=-1, keepdim=True)).to(bf)
    gv = rn(T, gH, dv).to(bf)
    if gates == "uniform":
        a = 0.9 + 0.1 * torch.rand(T, gH, generator=g, device="cuda")
        b = torch.rand(T, gH, generator=g, device="cuda")
    else:
        a = torch.sigmoid(3.0 + 0.5 * rn(T, gH))
        b = torch.sigmoid(rn(T, gH))
    out = dict(q=q, k=k, v=v, gq=gq, gk=gk, gv=gv, a=a.contiguous(), b=b.contiguous())
    out["root_state"] = None if root_std is None else (root_std * rn(R, gH, dv, dk)).contiguous()
    return out


def depth_of(parent):
    parent = np.asarray(parent)
    d = np.zeros(len(parent), np.int64)
    for s in range(len(parent)):
        if parent[s] >= 0:
            d[s] = d[parent[s]] + 1
    return int(d.max())


def wl_meta_of(parent, seg_len, H, Hkv, D, gH, dk, dv):
    return dict(parent=np.asarray(parent, np.int32), seg_len=np.asarray(seg_len, np.int32),
                T=int(np.sum(seg_len)), S=len(parent), depth=depth_of(parent), H=H, Hkv=Hkv, D=D,
                gH=gH, dk=dk, dv=dv)


# --------------------------------------------------------------- CPU baseline

def cpu_baseline(wl, threads):
    import oracle

    oracle.set_threads(threads, "f32")
    t0 = time.perf_counter()
    o, _ = oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, prec="f32")
    go, _, _ = oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b,
                          root_state=wl.root_state, prec="f32")
    dt = time.perf_counter() - t0
    return dt, o, go


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-workloads", action="store_true", help="headline workload only")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the block-piece, mixer and stack legs (kernel profiles of the step)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache and measured-peak passes (counter runs of the warm step)")
    ap.add_argument("--only", default=None, help="time just this workload (profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="finish with three plain 512 MiB device copies (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the hot path runs on one GPU (got --gpus {args.gpus}); "
              "sharding across GPUs is described in the design notes, not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tree_structured_decision_amd import metrics
    from tree_structured_decision_amd import workloads as W

    torch.cuda.set_device(0)
    log(f"device: {torch.cuda.get_device_name(0)}")

    if args.only:
        run_one(args.only, args.steps, args.warmup)
        calib_copy(args.calib_copy)
        return

    # ---------------- headline: one decision request
    wl = W.one_request()
    meta = wl_meta_of(wl.parent, wl.seg_len, wl.H, wl.Hkv, wl.D, wl.gH, wl.dk, wl.dv)
    r = Runner(meta, tensors_from_numpy(wl), graph=False)
    log(f"headline {wl.name}: T={wl.T} S={wl.S}; warmup {args.warmup}, steps {args.steps}")
    res = time_runner(r, args.steps, args.warmup)
    import torch
    cold = None
    if not args.no_cold:
        evict = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = time_runner(r, max(10, args.steps // 2), 2, evict=evict)
        del evict
    T = wl.T
    fl, ab = attn_work(wl.parent, wl.seg_len, wl.H, wl.Hkv, wl.D, 2)
    gb = gdn_work(wl.parent, wl.seg_len, wl.gH, wl.dk, wl.dv, 2, wl.root_state is not None)
    attn_ach = fl / res["attn_mean"]
    gdn_ach = gb / res["gdn_mean"]
    kernels = {
        "fork_attn_forward": dict(mean_us=res["attn_mean"] * 1e6, p50_us=res["attn_p50"] * 1e6,
                                  algorithmic_flop=fl, algorithmic_bytes=ab,
                                  achieved_tflops=attn_ach / 1e12,
                                  mfma_frac=attn_ach / PEAK_BF16_MFMA),
        "gdn_fork_forward": dict(mean_us=res["gdn_mean"] * 1e6, p50_us=res["gdn_p50"] * 1e6,
                                 algorithmic_bytes=gb, achieved_gbs=gdn_ach / 1e9,
                                 hbm_frac=gdn_ach / PEAK_HBM),
    }
    if res["attn_mean"] >= res["gdn_mean"]:
        tr = measured_traffic("fork_attn_forward")
        roof = dict(kernel="fork_attn_forward", bound="mfma", achieved=attn_ach / 1e12,
                    peak=PEAK_BF16_MFMA / 1e12, unit="TFLOP/s", frac=attn_ach / PEAK_BF16_MFMA,
                    traffic=None if tr is None else tr["bytes"])
    else:
        tr = measured_traffic("gdn_fork_forward")
        roof = dict(kernel="gdn_fork_forward", bound="hbm", achieved=gdn_ach / 1e9,
                    peak=PEAK_HBM / 1e9, unit="GB/s", frac=gdn_ach / PEAK_HBM,
                    traffic=None if tr is None else tr["bytes"])
    roof["algorithmic_per_launch"] = fl if roof["bound"] == "mfma" else gb
    roof["launches"] = (["fork_attn_kernel", "fork_attn_merge_kernel"] if roof["bound"] == "mfma" else
                        ["gdn_prep_kernel", "gdn_coop_kernel", "gdn_scan_kernel"])
    roof["note"] = ("one call of the layer, timed with HIP events on its stream; its kernels' "
                    "rocprofv3 averages are in profiles/one_request_kernels.md")
    kernels["fork_attn_forward"]["hbm_traffic_bytes"] = (measured_traffic("fork_attn_forward") or {}).get("bytes")
    kernels["gdn_fork_forward"]["hbm_traffic_bytes"] = (measured_traffic("gdn_fork_forward") or {}).get("bytes")

    # fidelity + CPU baseline (the float32 oracle serves both)
    o_gpu = r.o[:T].float().cpu().numpy()
    go_gpu = r.go[:T].float().cpu().numpy()
    cpu = None
    fid = None
    if not args.no_cpu:
        threads = min(len(os.sched_getaffinity(0)), 16)
        log(f"cpu baseline: fp32 oracle, {threads} threads")
        dt, o_ref, go_ref = cpu_baseline(wl, threads)
        cpu = dict(value=T / dt, unit="tokens/s", cores=threads, kind="oracle",
                   sample=f"the whole headline request (T={T}, both layers), fp32 oracle, "
                          f"{dt:.2f} s wall")
        fid = dict(attention=metrics.decision_fidelity(o_gpu, o_ref, wl.w_attn, wl.parent, wl.seg_len),
                   gdn=metrics.decision_fidelity(go_gpu, go_ref, wl.w_gdn, wl.parent, wl.seg_len),
                   reference="float32 oracle")

    n_opt, opt_tok, iso_tok = tree_rates(wl.parent, wl.seg_len)
    step_s = res["ms_per_step"] * 1e-3
    rates = dict(options=n_opt, option_tokens_per_s=opt_tok / step_s,
                 isolated_equivalent_tokens_per_s=iso_tok / step_s, us_per_option=step_s / n_opt * 1e6,
                 note="per step (wall); isolated-equivalent = sum over options of root-to-option path length")
    peaks = None
    if not args.no_cold:
        peaks = measured_peaks()
        if roof["bound"] == "mfma":
            roof["frac_measured_peak"] = roof["achieved"] / peaks["bf16_gemm_tflops"]
        else:
            roof["frac_measured_peak"] = roof["achieved"] / peaks["copy_gbs"]
    out = {
        "metric": METRIC,
        "value": T / (res["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one decision request: prefix 2048 + 16 options of 16-48 tokens; "
                               "attention 16 q / 2 kv heads, head_dim 128; Gated DeltaNet 16 heads, "
                               "dk = dv = 128",
                   "tokens": T, "segments": wl.S, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "layer_pair_p50_us": res["pair_p50"] * 1e6,
        "layer_pair_p95_us": res["pair_p95"] * 1e6,
        "fidelity": fid,
        "rates": rates,
        "cold_cache": None if cold is None else dict(
            pair_p50_us=cold["pair_p50"] * 1e6, attn_p50_us=cold["attn_p50"] * 1e6,
            gdn_p50_us=cold["gdn_p50"] * 1e6,
            note="512 MiB written between steps (outside the kernel events) to evict the L2 and "
                 "the Infinity Cache"),
        "measured_peaks": peaks,
    }
    if not args.no_extras:
        out["block_ops"] = {"one_request": block_ops(wl, r.sess)}
        out["mixers"] = {"one_request": mixer_ops(wl, r.sess)}
        st, st_inputs = stack_ops(wl, r.sess)
        if not args.no_cpu:
            st["fidelity"], st["fp8_fidelity"] = cpu_stack_fidelity(wl, st_inputs)
        out["stack"] = {"one_request": st}
    if not args.no_workloads:
        out["workloads"] = all_workloads(max(5, args.steps // 5), 3)
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


def build_workload(name):
    """(meta dict, device tensors, graph?) of a named workload."""
    from tree_structured_decision_amd import workloads as W

    if name in ("tiny_one_level", "one_request", "agent_history"):
        wl = W.WORKLOADS[name]()
        meta = wl_meta_of(wl.parent, wl.seg_len, wl.H, wl.Hkv, wl.D, wl.gH, wl.dk, wl.dv)
        meta["root_state"] = wl.root_state is not None
        return meta, tensors_from_numpy(wl), False, wl.dtype
    if name == "wide_options":
        parent, seg_len = W.tree_one_level(8192, [8] * 256)
        meta = wl_meta_of(parent, seg_len, 32, 4, 128, 16, 128, 128)
        t = tensors_on_device(name, parent, seg_len, 32, 4, 128, 16, 128, 128, 1003, "uniform", None)
        return meta, t, False, "bf16"
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
        meta = wl_meta_of(parent, seg_len, wl.H, wl.Hkv, wl.D, wl.gH, wl.dk, wl.dv)
        meta["ctx"] = (np.zeros(len(parent), np.int32), np.where(roots, P, 0).astype(np.int32), P)
        meta["root_state"] = True
        full = tensors_from_numpy(wl)
        t = {n: full[n][P:].contiguous() for n in ("q", "k", "v", "gq", "gk", "gv", "a", "b")}
        t["kc"], t["vc"] = full["k"][:P].contiguous(), full["v"][:P].contiguous()
        t["root_state"] = full["root_state"].expand(int(roots.sum()), -1, -1, -1).contiguous()
        return meta, t, False, wl.dtype
    if name == "request_mix":
        rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 5))
        parent, seg_len = W.request_mix_tree(rng)
        meta = wl_meta_of(parent, seg_len, 16, 2, 128, 16, 128, 128)
        t = tensors_on_device(name, parent, seg_len, 16, 2, 128, 16, 128, 128, 1005, "sigmoid", None)
        return meta, t, True, "bf16"
    raise ValueError(name)


def workload_report(name, meta, res, graph, dtype):
    elt = 2 if dtype == "bf16" else 4
    ctx = meta.get("ctx")
    fl, ab = attn_work(meta["parent"], meta["seg_len"], meta["H"], meta["Hkv"], meta["D"], elt,
                       ctx_len=None if ctx is None else ctx[1], ctx_rows=0 if ctx is None else ctx[2])
    gb = gdn_work(meta["parent"], meta["seg_len"], meta["gH"], meta["dk"], meta["dv"], elt,
                  meta.get("root_state", False))
    peak = PEAK_BF16_MFMA if dtype == "bf16" else PEAK_F32_MFMA
    roof_t = max(fl / peak, ab / PEAK_HBM) + gb / PEAK_HBM
    pair = res["pair_p50"]
    rep = dict(tokens=meta["T"], segments=meta["S"], graph=graph,
               stream_tokens_per_s=meta["T"] / (res["ms_per_step"] * 1e-3),
               layer_pair_p50_us=pair * 1e6,
               layer_pair_tokens_per_s=meta["T"] / pair,
               pair_roofline_frac=roof_t / pair)
    if not graph:
        rep.update(attn_p50_us=res["attn_p50"] * 1e6, gdn_p50_us=res["gdn_p50"] * 1e6,
                   attn_frac=max(fl / peak, ab / PEAK_HBM) / res["attn_p50"],
                   attn_tflops=fl / res["attn_p50"] / 1e12,
                   gdn_hbm_frac=(gb / PEAK_HBM) / res["gdn_p50"])
    return rep


def all_workloads(steps, warmup):
    import torch

    rep = {}
    for name in ("tiny_one_level", "one_request", "wide_options", "agent_history",
                 "agent_history_resume", "request_mix"):
        log(f"workload {name}")
        meta, t, graph, dtype = build_workload(name)
        r = Runner(meta, t, graph)
        res = time_runner(r, steps, warmup)
        rep[name] = workload_report(name, meta, res, graph, dtype)
        log(f"  {rep[name]}")
        r.sess.close()
        del r, t
        torch.cuda.empty_cache()
    return rep


def run_one(name, steps, warmup):
    meta, t, graph, dtype = build_workload(name)
    r = Runner(meta, t, graph)
    res = time_runner(r, steps, warmup)
    print(json.dumps({name: workload_report(name, meta, res, graph, dtype)}), flush=True)


if __name__ == "__main__":
    main()
