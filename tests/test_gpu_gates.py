"""Gated DeltaNet at the gates' extreme values, against the oracle (the
token recurrence S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T):

- a = 0 at scattered tokens: the state is forgotten there. The chunked form
  works with decay ratios exp(g_i - g_j) of prefix sums g of log a, which a
  zero gate must turn into exact zeros rather than -inf - (-inf).
- a = 1 and b = 0 everywhere: the state never changes, so every output is
  scale * S_root q_t and every start and end state is the root's.
- a = 1 and b = 1 everywhere: the pure delta rule.

On trees with a multi-chunk root (at this size the chunk-cooperative kernel
takes it) and children, bf16 and fp32, with end states requested and without
(leaf siblings packed into shared chunks), and with FP8 inputs. The bar is
the one of the other parity tests (plain max-abs on o where |ref| < 8, and on
the fp32 states)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, log, oracle_gdn, run_hip
from tests.test_gpu_gdn_fp8 import oracle_on, run_fp8, session_for
from tree_structured_decision_amd import workloads as W

pytestmark = pytest.mark.gpu

# a root of five chunks with a ragged tail, two inner children, leaf siblings
PARENT = np.array([-1, 0, 0, 1, 1, 1, 2, 2, -1, 8], np.int32)
SEG_LEN = np.array([301, 70, 9, 5, 17, 40, 3, 64, 33, 12], np.int32)


def gated(dtype, gates, seed, dk=128, gH=4, root_std=0.5):
    wl = W.make_workload("gates", dtype, PARENT, SEG_LEN, H=4, Hkv=2, D=64, gH=gH, dk=dk, dv=dk,
                         gates="sigmoid", root_state_std=root_std, seed=seed)
    rng = np.random.default_rng(seed)
    a, b = wl.a.copy(), wl.b.copy()
    if gates == "reset":
        # zero gates on ~8 % of the (token, head) pairs, on a chunk's first
        # and last row and on a segment's first token among them
        a[rng.random(a.shape) < 0.08] = 0.0
        a[[0, 63, 64, 127, 301, 371], :] = 0.0
    elif gates == "hold":
        a[:] = 1.0
        b[:] = 0.0
    elif gates == "delta":
        a[:] = 1.0
        b[:] = 1.0
    else:
        raise ValueError(gates)
    return dataclasses.replace(wl, a=a, b=b)


def check(wl, got, ref, final):
    go, s0, s1 = ref
    check_close("gdn.o", got["go"], go, wl.dtype)
    check_close("gdn.start_state", got["s0"], s0, wl.dtype, kind="f32")
    if final:
        check_close("gdn.final_state", got["s1"], s1, wl.dtype, kind="f32")


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("bf16", 64), ("f32", 32)])
@pytest.mark.parametrize("gates", ["reset", "hold", "delta"])
@pytest.mark.parametrize("final", [True, False])
def test_extreme_gates(dtype, dk, gates, final):
    wl = gated(dtype, gates, seed=100 + dk + 10 * ["reset", "hold", "delta"].index(gates), dk=dk)
    log(f"gates={gates} {dtype} dk={dk} final={final}: T={wl.T} S={wl.S}")
    got = run_hip(wl, attn=False, final=final)
    check(wl, got, oracle_gdn(wl), final)
    if gates == "hold":
        # the state is the root's throughout: o_t = scale * S_root q_t exactly
        # as the oracle has it, and every start state is its root's state
        p = np.asarray(wl.parent)
        root = np.zeros(wl.S, np.int64)
        for s in range(wl.S):
            root[s] = s if p[s] < 0 else root[p[s]]
        rid = np.cumsum(p < 0) - 1
        want = wl.root_state[rid[root]].astype(np.float64)
        np.testing.assert_array_equal(got["s0"], want)


@pytest.mark.parametrize("gates", ["reset", "hold"])
def test_extreme_gates_fp8(gates):
    wl = gated("bf16", gates, seed=91, dk=128)
    sess = session_for(wl)
    got, qkv = run_fp8(wl, sess, final=True)
    sess.close()
    check(wl, got, oracle_on(wl, qkv), True)
