"""Tree attention with the online softmax under stress, against the oracle
(fp64 softmax over each row's visible keys):

- rising scores (each 32-key half raises a row's max past the rescale
  margin): the running max is raised at every half and the accumulators are
  rescaled each time;
- falling scores: the max is set by a row's first keys and never raised;
- large random scores: near one-hot weights.

On a prefix of several key tiles with options (split query tiles and their
merge included), bf16 and fp32, D 64 and 128, log-sum-exps up to ~450; and
with FP8 scores (the oracle on the decoded queries and keys) at log-sum-exps
up to ~60.

The bars follow the arithmetic. fp32: a score error ds moves a softmax
average by at most 2 max|v| max|ds| and the log-sum-exp by max|ds|, and a
D-term fp32 dot product errs by about sqrt(D) 2^-24 sum_i |q_i k_i| <= sqrt(D)
2^-24 |q| |k|: 1e-4 + 2 max|v| sqrt(D) 2^-24 scale max|q| max|k| on o (~3e-3
at these scores). bf16: the kernel rounds the weights p to bf16 (relative
2^-9) for the value product and sums the rounded weights, so o is an exact
average under weights perturbed by at most 2^-9 each; to first order that
moves o by at most 2^-9 max_j |v_j - o| <= 2^-8 max|v|, which near-one-hot
rows reach, and the output's own bf16 rounding adds half an ulp of o: the
bar on o is half an ulp + 2^-8 max|v| + 1e-3 elementwise (max-abs 2e-2, the
bar of the workload tests, can be exceeded here by up to that 2^-8 max|v|
term), 2e-2 on the log-sum-exp."""
import dataclasses

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import log, oracle_attn, run_hip
from tests.test_gpu_attn_fp8 import run_qk8, session_for
from tree_structured_decision_amd import workloads as W

pytestmark = pytest.mark.gpu

PARENT = np.array([-1, 0, 0, 0, 1], np.int32)
SEG_LEN = np.array([700, 90, 33, 5, 70], np.int32)


def stressed(dtype, D, pattern, seed, mag=1.0):
    """mag scales the score magnitudes (the keys)."""
    wl = W.make_workload("softmax", dtype, PARENT, SEG_LEN, H=8, Hkv=2, D=D, gH=2, dk=32, dv=32,
                         gates="sigmoid", root_state_std=None, seed=seed)
    q, k = wl.q.copy(), wl.k.copy()
    T = wl.T
    scale = 1.0 / np.sqrt(D)
    if pattern in ("rising", "falling"):
        # score(t, j) ~ step * pos(j): step * 32 keys * log2(e) is past the
        # rescale margin of 8 (log2 units) at mag >= 1/8
        step = 0.5 * mag
        pos = np.arange(T, dtype=np.float64)
        if pattern == "falling":
            pos = T - pos
        q[..., 0] = 1.0
        k[..., 0] = step * pos[:, None] / scale
        q[..., 1:] *= 0.1
    elif pattern == "large":
        q *= 6.0
        k *= 6.0 * mag
    else:
        raise ValueError(pattern)
    if dtype == "bf16":
        q, k = W.round_bf16(q), W.round_bf16(k)
    return dataclasses.replace(wl, q=q.astype(np.float32), k=k.astype(np.float32))


def score_bound(wl):
    """scale * max|q| * max|k| >= sum_i |q_i k_i| * scale for every pair."""
    qn = np.linalg.norm(wl.q.astype(np.float64), axis=-1).max()
    kn = np.linalg.norm(wl.k.astype(np.float64), axis=-1).max()
    return qn * kn / np.sqrt(wl.D)


def half_ulp_bf16(x):
    m = np.maximum(np.abs(x), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(m)) - 8)


def check(name, got, ref, tol):
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    worst = float((err - tol).max())
    log(f"  {name}: max-abs {float(err.max()):.3e}, worst margin to the bar {-worst:.3e}")
    assert worst <= 0, f"{name}: error exceeds the bar by {worst}"


def check_bf16(name, o, lse, o_ref, lse_ref, vmax):
    check(f"{name} o", o, o_ref, half_ulp_bf16(o_ref) + 2.0**-8 * vmax + 1e-3)
    check(f"{name} lse", lse, lse_ref, 2e-2)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("pattern", ["rising", "falling", "large"])
def test_softmax_stress(dtype, D, pattern):
    wl = stressed(dtype, D, pattern, seed=200 + D + len(pattern))
    o, lse = oracle_attn(wl)
    vmax = float(np.abs(wl.v).max())
    log(f"{pattern} {dtype} D={D}: T={wl.T}, lse range [{lse.min():.1f}, {lse.max():.1f}]")
    for split in (True, False):
        got = run_hip(wl, gdn=False, split=split)
        if wl.dtype == "bf16":
            check_bf16(f"attn (split={split})", got["o"], got["lse"], o, lse, vmax)
            continue
        ds = np.sqrt(wl.D) * 2.0**-24 * score_bound(wl)  # bound on a score's fp32 error
        check(f"attn o (split={split})", got["o"], o, 1e-4 + 2 * vmax * ds)
        check(f"attn lse (split={split})", got["lse"], lse, 1e-4 + 2 * ds)


@pytest.mark.parametrize("pattern", ["rising", "falling", "large"])
def test_softmax_stress_fp8_scores(pattern):
    """FP8 scores (per-row E4M3 queries and keys) at scores up to ~60 nats.
    (The FP8 matrix cores' dot products are less exact than fp32 when one
    product dominates the others: the log-sum-exp error grows in proportion
    to the score, ~9e-5 of it, so larger scores exceed these bars.)"""
    wl = stressed("bf16", 128, pattern, seed=300 + len(pattern), mag=0.125)
    sess = session_for(wl)
    o, lse, qd, kd = run_qk8(wl, sess)
    sess.close()
    o_ref, lse_ref = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v)
    log(f"{pattern} FP8 scores: lse range [{lse_ref.min():.1f}, {lse_ref.max():.1f}]")
    check_bf16("qk8", o, lse, o_ref, lse_ref, float(np.abs(wl.v).max()))
