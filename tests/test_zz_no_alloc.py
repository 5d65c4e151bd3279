"""fork_attn_forward_noalloc: the attention entry point that allocates
nothing (its split-tile partial results live in a scratch array compiled
into the library, one copy per GPU). Checked through the C ABI against
fork_attn_forward with a caller workspace, on two calls in a row, the second
with a smaller tree, and against the oracle's bar."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_helpers import TOL, check_close, log, oracle_attn
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

pytestmark = pytest.mark.gpu


def small_split_tree():
    rng = np.random.default_rng(11)
    parent, seg_len = W.random_tree(rng, 12, 300, max_depth=3, roots=2)
    return W.make_workload("noalloc-small", "bf16", parent, seg_len, H=16, Hkv=2, D=128, gH=2, dk=32,
                           dv=32, gates="sigmoid", root_state_std=None, seed=12)


def run_both(sess, wl, d):
    """fork_attn_forward_ctx with the session's workspace, then the no-alloc call."""
    out = {}
    for mode in ("workspace", "noalloc"):
        o = torch.full_like(d["q"], float("nan"))
        lse = torch.full((wl.T, wl.H), float("nan"), device="cuda")
        if mode == "workspace":
            sess.attention(d["q"], d["k"], d["v"], o, lse)
        else:
            B.fork_attn_forward_noalloc(sess.meta, d["q"], d["k"], d["v"], None, None, o, lse, wl.H, wl.Hkv,
                                        wl.D, 0.0, B.FORK_BF16)
        torch.cuda.synchronize()
        out[mode] = (o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    return out


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big, small = W.one_request(), small_split_tree()
    assert small.T < big.T
    # one session sized for the larger tree; the smaller is built into the same blob
    caps = caps_for(big.parent, big.seg_len, big.H // big.Hkv, kv_heads=big.Hkv, depth_cap=3)
    sess = ForkSession(**caps, D=big.D, gH=2, dk=32, dv=32)
    for wl in (big, small):
        d = to_device(wl, "cuda")
        sess.build(wl.parent, wl.seg_len)
        assert sess.meta.num_attn_parts > 0, "the case must split query tiles (use the scratch)"
        need = sess.meta.num_attn_parts * wl.Hkv * (256 * wl.D * 2 + 256 * 4)
        log(f"{wl.name}: T={wl.T} S={wl.S}, {sess.meta.num_attn_merges} split tiles, "
            f"{sess.meta.num_attn_parts} parts, {need / 2**20:.1f} MiB of scratch")
        got = run_both(sess, wl, d)
        (ow, lw), (on, ln) = got["workspace"], got["noalloc"]
        check_close(f"{wl.name} noalloc o vs workspace o", on, ow, "bf16")
        check_close(f"{wl.name} noalloc lse vs workspace lse", ln, lw, "bf16", kind="f32")
        assert np.array_equal(on, ow) and np.array_equal(ln, lw), "same kernels, same plan: expected bitwise"
        o_ref, lse_ref = oracle_attn(wl)
        check_close(f"{wl.name} noalloc o vs oracle", on, o_ref, "bf16")
        check_close(f"{wl.name} noalloc lse vs oracle", ln, lse_ref, "bf16", kind="f32")
        assert sess.check() == 0
    sess.close()


def test_noalloc_rejects_a_plan_beyond_the_scratch_without_launching():
    wl = W.one_request()
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv)
    sess = ForkSession(**caps, D=wl.D)
    sess.build(wl.parent, wl.seg_len)
    torch.cuda.synchronize()
    m = B.fork_meta()
    ctypes.memmove(ctypes.byref(m), ctypes.byref(sess.meta), ctypes.sizeof(m))
    m.num_attn_parts = 4096  # 4096 x 2 slots of 65 KB > 64 MiB
    d = to_device(wl, "cuda")
    o = torch.full_like(d["q"], float("nan"))
    with pytest.raises(B.ForkError) as e:
        B.fork_attn_forward_noalloc(m, d["q"], d["k"], d["v"], None, None, o, None, wl.H, wl.Hkv, wl.D, 0.0,
                                    B.FORK_BF16)
    assert e.value.status == -5 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all()
    sess.close()
