"""Helpers for the GPU parity tests: run the HIP path on a workload-shaped
input and compare with the oracle under the stated tolerances.

Tolerances (max over every output element):
* fp32 inputs and outputs: |gpu - oracle| <= 1e-4;
* bf16 inputs and outputs, fp32 accumulation: plain |gpu - oracle| <= 2e-2 on
  every element whose exact value is below 8 in magnitude. At |value| >= 8 half
  a bf16 ulp is 1/32 > 2e-2, so a correctly rounded result could not meet the
  plain bar there: those elements get 2e-2 plus half a bf16 ulp of the value,
  and their count and largest error in bf16 ulps are printed beside the
  plain max-abs; fp32 outputs of bf16 runs (log-sum-exp, states):
  |gpu - oracle| <= 2e-2.
"""
import numpy as np
import torch

import oracle
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg):
    print(msg, flush=True)


def run_hip(wl, *, attn=True, gdn=True, sess=None, final=True, device="cuda", split=True):
    """Run the requested layers on the GPU; returns numpy float64 outputs.
    split: plan split query tiles (kv_heads given) or not."""
    own = sess is None
    if own:
        caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv if split else 0)
        sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv, device=device)
    d = to_device(wl, device)
    sess.build(wl.parent, wl.seg_len)
    out = {}
    if attn:
        o = torch.full_like(d["q"], float("nan"))
        lse = torch.full((wl.T, wl.H), float("nan"), device=device)
        sess.attention(d["q"], d["k"], d["v"], o, lse)
        out["o"], out["lse"] = o, lse
    if gdn:
        go = torch.full((wl.T, wl.gH, wl.dv), float("nan"), device=device, dtype=d["gq"].dtype)
        st0 = torch.full((wl.S, wl.gH, wl.dv, wl.dk), float("nan"), device=device)
        st1 = torch.full_like(st0, float("nan")) if final else None
        sess.gdn(d["gq"], d["gk"], d["gv"], d["a"], d["b"], go, st0, st1,
                 root_state=d["root_state"])
        out["go"], out["s0"] = go, st0
        if final:
            out["s1"] = st1
    torch.cuda.synchronize()
    res = {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}
    if own:
        sess.close()
    return res


def check_close(name, got, ref, dtype, kind="out", rows=None):
    """kind: 'out' for outputs stored in the workload dtype, 'f32' for fp32
    outputs (lse, states). Returns the plain max-abs error."""
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{name}: non-finite values (unwritten output?)"
    assert np.isfinite(ref).all(), f"{name}: non-finite reference values (unselected rows?)"
    tol = TOL[dtype]
    err = np.abs(got - ref)
    m = float(err.max()) if err.size else 0.0
    if kind == "out" and dtype == "bf16":
        big = np.abs(ref) >= 8.0
        small_max = float(err[~big].max()) if (~big).any() else 0.0
        msg = f"  {name}: max-abs {m:.3e} (|ref| < 8: {small_max:.3e}, tol {tol:.0e}) over {err.size} values"
        if big.any():
            ulp = 2.0 * metrics.bf16_half_ulp(ref[big])
            in_ulps = err[big] / ulp
            msg += f"; {int(big.sum())} values with |ref| >= 8, max error {float(in_ulps.max()):.3f} bf16 ulp"
            excess = float((err[big] - ulp / 2).max())
            assert excess <= tol, f"{name}: error at |ref| >= 8 exceeds 2e-2 + half a bf16 ulp by {excess - tol}"
        log(msg)
        assert small_max <= tol, f"{name}: max error {small_max} > {tol} where |ref| < 8"
    else:
        log(f"  {name}: max-abs {m:.3e} (tol {tol:.0e}) over {err.size} values")
        assert m <= tol, f"{name}: max error {m} > {tol}"
    return m


def oracle_attn(wl, tok_select=None):
    return oracle.attention(wl.parent, wl.seg_len, wl.q, wl.k, wl.v, tok_select=tok_select)


def oracle_gdn(wl, seg_select=None):
    return oracle.gdn(wl.parent, wl.seg_len, wl.gq, wl.gk, wl.gv, wl.a, wl.b,
                      root_state=wl.root_state, seg_select=seg_select)
