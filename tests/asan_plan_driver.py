"""Driver for the host AddressSanitizer test (run by tests/test_host_asan.py in
a child process with the sanitizer runtime preloaded; not collected by
pytest). It loads the library build whose host code is instrumented (path in
argv[1]) and runs every host-only entry point of the C ABI that plans or
validates: the capacity queries and the metadata plan (with and without
resumed contexts) on the workload trees and on many random trees, at exact
capacities (no slack in any buffer) and with key-range splitting, plus the
rejection paths (malformed trees, capacities exceeded, short staging
buffers, the FP8 Gated DeltaNet entry point's argument checks). Nothing here touches a GPU. Exits 0 when every call behaved; the
sanitizer aborts the process on the first invalid memory access."""
import sys

import numpy as np

from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import workloads as W

CODE = {name: code for code, name in B.STATUS.items()}


def plan(parent, seg_len, gqa=8, kv_heads=0, depth_cap=None, ctx=None, t_slack=0, s_slack=0):
    parent = np.ascontiguousarray(parent, np.int32)
    seg_len = np.ascontiguousarray(seg_len, np.int32)
    depth = np.zeros(len(parent), np.int32)
    for s, p in enumerate(parent):
        depth[s] = 0 if p < 0 else depth[p] + 1
    ctx_cap = 0 if ctx is None else int((ctx[0] + ctx[1]).max(initial=0))
    caps = B.make_caps(int(seg_len.sum()) + t_slack, len(parent) + s_slack,
                       int(depth.max()) if depth_cap is None else depth_cap, gqa, kv_heads, ctx_cap)
    _, stg = B.fork_meta_size(caps)
    staging = np.zeros(stg // 4, np.int32)  # exactly the size asked for
    if ctx is None:
        meta, up = B.fork_meta_plan(parent, seg_len, caps, staging)
    else:
        meta, up = B.fork_meta_plan_ctx(parent, seg_len, np.ascontiguousarray(ctx[0], np.int32),
                                        np.ascontiguousarray(ctx[1], np.int32), caps, staging)
    assert 0 < up <= staging.nbytes
    return meta


def expect_error(fn, status):
    try:
        fn()
    except B.ForkError as e:
        assert e.status == status, (e.status, status, str(e))
        return
    raise AssertionError("call was expected to fail")


def main():
    import ctypes
    ctypes.CDLL(None).__asan_init  # the sanitizer runtime is loaded in this process
    B.LIB_PATH = sys.argv[1]
    n = 0
    # workload trees, every GQA shape the kernels take, with and without splitting
    for make in (W.tiny_one_level, W.one_request, W.wide_options, W.agent_history):
        wl = make()
        for gqa, kvh in ((wl.H // wl.Hkv, 0), (wl.H // wl.Hkv, wl.Hkv), (1, 4), (64, 2), (256, 1)):
            plan(wl.parent, wl.seg_len, gqa, kvh)
            n += 1
    rng = np.random.Generator(np.random.PCG64(W.SEED_BASE + 5))
    parent, seg_len = W.request_mix_tree(rng)
    for gqa, kvh in ((8, 2), (8, 0)):
        plan(parent, seg_len, gqa, kvh)
        plan(parent, seg_len, gqa, kvh, depth_cap=3, t_slack=1000, s_slack=17)
        n += 2
    # random trees: ragged lengths, several roots, deep chains, resumed contexts
    rng = np.random.default_rng(7)
    for it in range(300):
        S = int(rng.integers(1, 60))
        roots = int(rng.integers(1, min(S, 4) + 1))
        p, L = W.random_tree(rng, S, int(rng.choice([1, 8, 70, 300])), max_depth=int(rng.integers(2, 8)),
                             roots=roots)
        gqa = int(rng.choice([1, 2, 3, 8, 32, 64]))
        kvh = int(rng.choice([0, 1, 2]))
        ctx = None
        if it % 3 == 0:
            cl = np.where(p < 0, rng.integers(0, 500, S), 0).astype(np.int32)
            cs = np.where(cl > 0, rng.integers(0, 1000, S), 0).astype(np.int32)
            ctx = (cs, cl)
        plan(p, L, gqa, kvh, ctx=ctx, t_slack=int(rng.integers(0, 3)) * 64)
        n += 1
    chain = np.arange(-1, 199, dtype=np.int32)
    plan(chain, np.full(200, 3, np.int32), 4, 2)
    # rejections
    p = np.array([-1, 0, 1], np.int32)
    L = np.array([5, 6, 7], np.int32)
    expect_error(lambda: plan(np.array([-1, 2, 0], np.int32), L), CODE["FORK_E_TREE"])
    expect_error(lambda: plan(p, np.array([5, 0, 7], np.int32)), CODE["FORK_E_TREE"])
    expect_error(lambda: plan(p, L, t_slack=-1), CODE["FORK_E_CAPACITY"])
    expect_error(lambda: plan(p, L, depth_cap=1), CODE["FORK_E_CAPACITY"])
    caps = B.make_caps(18, 3, 2, 8)
    _, stg = B.fork_meta_size(caps)
    expect_error(lambda: B.fork_meta_plan(p, L, caps, np.zeros(stg // 4 - 1, np.int32)), CODE["FORK_E_WORKSPACE"])
    big = B.make_caps(1 << 29, 1 << 20, 8, 256, 2)
    expect_error(lambda: B.fork_meta_size(big), CODE["FORK_E_CAPACITY"])
    bad_ctx = (np.array([0, 0, 0], np.int32), np.array([0, 4, 0], np.int32))
    expect_error(lambda: plan(p, L, ctx=bad_ctx), CODE["FORK_E_TREE"])
    # argument checks of the FP8 Gated DeltaNet entry point, which run before
    # any launch: a plan-only descriptor given a stand-in blob address (never
    # dereferenced on these paths), integer stand-ins for the device pointers
    meta = plan(p, L)
    meta.dev = 1 << 20
    meta.dev_bytes = 1 << 40
    a16 = 1 << 21
    fp8 = lambda q8=a16, qs=a16, dk=128: B.gdn_fork_forward_fp8(meta, q8, qs, a16, a16, a16, a16, a16, a16, None,
                                                                 a16, a16, None, 4, dk, dk, 1.0, stream=0)
    expect_error(lambda: fp8(qs=None), CODE["FORK_E_ARG"])
    expect_error(lambda: fp8(dk=64), CODE["FORK_E_UNSUPPORTED"])
    expect_error(lambda: fp8(q8=a16 + 1), CODE["FORK_E_ARG"])
    # the decision readout's argument checks (same stand-ins)
    ro = lambda x=a16, C=64: B.fork_option_readout(meta, x, a16, C, a16, a16, B.FORK_BF16, stream=0)
    expect_error(lambda: ro(x=None), CODE["FORK_E_ARG"])
    expect_error(lambda: ro(C=12), CODE["FORK_E_UNSUPPORTED"])
    expect_error(lambda: ro(x=a16 + 8), CODE["FORK_E_ARG"])
    print(f"asan driver: {n} plans and 13 rejections checked", flush=True)


if __name__ == "__main__":
    main()
