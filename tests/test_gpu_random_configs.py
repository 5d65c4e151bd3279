"""Randomised parity: seeded random trees (1-60 segments, 1-4 roots, depth up
to 7, segments of 1 to 1500 tokens, up to 8000 tokens in all) under random
configurations (bf16 or fp32; D 64 or 128; GQA groups 1-8 with 1-4 kv heads;
Gated DeltaNet head size 32, 64 or 128 and 1-3 heads; sigmoid or uniform
gates; zero or given root states; end states requested or not, so leaf
siblings run packed or not; split query tiles planned or not), the
attention and Gated DeltaNet outputs, log-sum-exps and states against the
oracle, and for some bf16 cases the FP8-score attention and FP8 Gated
DeltaNet launches against the oracle on their decoded inputs. Every case is
reproducible from its seed; a failure names it and its configuration."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import check_close, log, oracle_attn, oracle_gdn, run_hip
from tests.test_gpu_attn_fp8 import run_qk8, session_for as attn8_session
from tests.test_gpu_gdn_fp8 import oracle_on, run_fp8, session_for as gdn8_session
from tree_structured_decision_amd import workloads as W

pytestmark = pytest.mark.gpu


def draw_case(case):
    rng = np.random.default_rng(10_000 + case)
    S = int(rng.integers(1, 60))
    roots = int(rng.integers(1, min(S, 4) + 1))
    parent, seg_len = W.random_tree(rng, S, int(rng.choice([3, 40, 150, 400, 1500])),
                                    max_depth=int(rng.integers(2, 8)), roots=roots)
    cfg = dict(dtype=str(rng.choice(["bf16", "bf16", "f32"])), D=int(rng.choice([64, 128])))
    cfg["H"], cfg["Hkv"] = [(4, 2), (8, 1), (16, 2), (6, 3), (12, 4), (2, 2)][int(rng.integers(0, 6))]
    cfg["dk"] = int(rng.choice([32, 64, 128])) if cfg["dtype"] == "f32" else int(rng.choice([64, 128, 128]))
    cfg["gH"] = int(rng.integers(1, 4))
    cfg["gates"] = str(rng.choice(["sigmoid", "uniform"]))
    cfg["root_std"] = None if rng.random() < 0.5 else 0.3
    cfg["final"] = bool(rng.random() < 0.5)
    cfg["split"] = bool(rng.random() < 0.7)
    cfg["fp8_attn"] = bool(rng.random() < 0.5)
    cfg["fp8_gdn"] = bool(rng.random() < 0.5)
    return parent, seg_len, cfg


def run_case(case):
    parent, seg_len, c = draw_case(case)
    if int(seg_len.sum()) > 8000:
        return False
    dt = c["dtype"]
    wl = W.make_workload("random", dt, parent, seg_len, H=c["H"], Hkv=c["Hkv"], D=c["D"], gH=c["gH"],
                         dk=c["dk"], dv=c["dk"], gates=c["gates"], root_state_std=c["root_std"], seed=case)
    log(f"case {case}: S={wl.S} T={wl.T} {c}")
    got = run_hip(wl, final=c["final"], split=c["split"])
    o, lse = oracle_attn(wl)
    check_close("attn.o", got["o"], o, dt)
    check_close("attn.lse", got["lse"], lse, dt, kind="f32")
    go, s0, s1 = oracle_gdn(wl)
    check_close("gdn.o", got["go"], go, dt)
    check_close("gdn.start_state", got["s0"], s0, dt, kind="f32")
    if c["final"]:
        check_close("gdn.final_state", got["s1"], s1, dt, kind="f32")
    if dt == "bf16" and c["D"] == 128 and c["fp8_attn"]:
        sess = attn8_session(wl, c["split"])
        o8, l8, qd, kd = run_qk8(wl, sess)
        sess.close()
        r8, rl8 = oracle.attention(wl.parent, wl.seg_len, qd, kd, wl.v)
        check_close("qk8.o", o8, r8, "bf16")
        check_close("qk8.lse", l8, rl8, "bf16", kind="f32")
    if dt == "bf16" and c["dk"] == 128 and c["fp8_gdn"]:
        sess = gdn8_session(wl)
        g8, qkv = run_fp8(wl, sess, final=c["final"])
        sess.close()
        ref = oracle_on(wl, qkv)
        check_close("gdn8.o", g8["go"], ref[0], "bf16")
        check_close("gdn8.start_state", g8["s0"], ref[1], "bf16", kind="f32")
    return True


@pytest.mark.parametrize("batch", range(4))
def test_random_configurations(batch):
    ran = sum(run_case(case) for case in range(1000 + 60 * batch, 1000 + 60 * (batch + 1)))
    assert ran > 30
