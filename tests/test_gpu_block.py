"""GPU parity of the fork-aware block pieces (rotary embedding at isolated
positions, causal depthwise convolution along isolated sequences) against the
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import check_close, log
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for

pytestmark = pytest.mark.gpu
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def tree_case(seed, n_seg=14, max_len=40, roots=2, ctx=True):
    rng = np.random.default_rng(seed)
    parent, seg_len = W.random_tree(rng, n_seg, max_len, max_depth=5, roots=roots)
    # some very short segments, so windows reach across several ancestors
    seg_len[rng.integers(0, n_seg, 4)] = rng.integers(1, 3, 4)
    S = len(parent)
    ctx_len = np.where(parent < 0, rng.integers(1, 300, S), 0).astype(np.int32) if ctx else None
    ctx_start = None if ctx_len is None else np.concatenate([[0], np.cumsum(ctx_len)[:-1]]).astype(np.int32)
    return rng, parent, seg_len.astype(np.int32), ctx_start, ctx_len


def session_for(parent, seg_len, ctx_start, ctx_len):
    C = 0 if ctx_len is None else int((ctx_start + ctx_len).max())
    sess = ForkSession(**caps_for(parent, seg_len, 8, ctx_cap=C))
    sess.build(parent, seg_len, ctx_start=ctx_start, ctx_len=ctx_len)
    return sess


@pytest.mark.parametrize("dtype,D,seed", [("f32", 64, 1), ("bf16", 128, 2), ("f32", 8, 3), ("bf16", 256, 4)])
def test_rope_parity(dtype, D, seed):
    rng, parent, seg_len, cs, cl = tree_case(seed)
    T = int(seg_len.sum())
    x = rng.standard_normal((T, 3, D)).astype(np.float32)
    if dtype == "bf16":
        x = W.round_bf16(x)
    sess = session_for(parent, seg_len, cs, cl)
    xd = torch.from_numpy(x).to("cuda", TORCH_DT[dtype])
    sess.rope(xd, theta=10000.0)
    torch.cuda.synchronize()
    ref = oracle.rope(parent, seg_len, x, theta=10000.0, ctx_len=cl)
    check_close(f"rope {dtype} D={D}", xd.float().cpu().numpy().astype(np.float64), ref, dtype)


def test_rope_long_positions():
    """Positions near 300k (a long resumed context): the angle is reduced in
    double precision, so the rotation stays accurate."""
    parent = np.array([-1, 0, 0], np.int32)
    seg_len = np.array([50, 20, 30], np.int32)
    cs, cl = np.array([0, 0, 0], np.int32), np.array([299_900, 0, 0], np.int32)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((100, 2, 128)).astype(np.float32)
    sess = session_for(parent, seg_len, cs, cl)
    xd = torch.from_numpy(x).cuda()
    sess.rope(xd, theta=10000.0)
    torch.cuda.synchronize()
    ref = oracle.rope(parent, seg_len, x, theta=10000.0, ctx_len=cl)
    check_close("rope at positions ~3e5", xd.cpu().numpy().astype(np.float64), ref, "f32")


@pytest.mark.parametrize("dtype,K,act,bias,state,seed", [
    ("f32", 4, 1, True, True, 5), ("f32", 2, 0, False, False, 6), ("bf16", 3, 1, True, False, 7),
    ("bf16", 4, 1, True, True, 10),
    ("bf16", 8, 1, False, True, 8), ("f32", 8, 0, True, True, 9)])
def test_conv_parity(dtype, K, act, bias, state, seed):
    rng, parent, seg_len, cs, cl = tree_case(seed, ctx=False)
    T, S = int(seg_len.sum()), len(parent)
    R = int((parent < 0).sum())
    C = 48
    x = rng.standard_normal((T, C)).astype(np.float32)
    if dtype == "bf16":
        x = W.round_bf16(x)
    w = (rng.standard_normal((C, K)) / np.sqrt(K)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32) if bias else None
    st = rng.standard_normal((R, C, K - 1)).astype(np.float32) if state else None
    sess = session_for(parent, seg_len, None, None)
    xd = torch.from_numpy(x).to("cuda", TORCH_DT[dtype])
    y = torch.full_like(xd, float("nan"))
    dev = lambda a: None if a is None else torch.from_numpy(a).cuda()
    sess.conv(xd, dev(w), y, bias=dev(b), conv_state=dev(st), act=act)
    torch.cuda.synchronize()
    ref = oracle.conv(parent, seg_len, x, w, bias=b, conv_state=st, act=act)
    check_close(f"conv {dtype} K={K} act={act}", y.float().cpu().numpy().astype(np.float64), ref, dtype)


def test_block_pieces_one_request_full():
    """The one-request tree at full size: rotary embedding of the attention
    q heads and the short convolution of the Gated DeltaNet q | k | v
    channels (3 x 16 x 128), bf16, whole outputs against the oracle."""
    wl = W.one_request()
    sess = ForkSession(**caps_for(wl.parent, wl.seg_len, 8))
    sess.build(wl.parent, wl.seg_len)
    q = torch.from_numpy(wl.q).to("cuda", torch.bfloat16)
    sess.rope(q)
    x = np.concatenate([wl.gq.reshape(wl.T, -1), wl.gk.reshape(wl.T, -1), wl.gv.reshape(wl.T, -1)], axis=1)
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((x.shape[1], 4)) / 2).astype(np.float32)
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    y = torch.full_like(xd, float("nan"))
    sess.conv(xd, torch.from_numpy(w).cuda(), y, act=1)
    torch.cuda.synchronize()
    check_close("rope(q) one request", q.float().cpu().numpy().astype(np.float64),
                oracle.rope(wl.parent, wl.seg_len, wl.q), "bf16")
    check_close("conv(q|k|v) one request", y.float().cpu().numpy().astype(np.float64),
                oracle.conv(wl.parent, wl.seg_len, x, w, act=1), "bf16")
