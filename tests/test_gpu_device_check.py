"""The device error word of a metadata blob (fork_meta_check).

Every kernel checks the blob's header against the capacities its launch was
made for before touching anything else. The failure cases are forced from the
host (the header words are overwritten between the build and the launch), so
every kernel still exits normally: it sets its bit and returns without
reading the tree or writing an output."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import log
from tree_structured_decision_amd import binding as B
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession, caps_for, to_device

pytestmark = pytest.mark.gpu

MH_MAGIC, MH_T = 0, 1


def setup():
    rng = np.random.default_rng(3)
    parent, seg_len = W.random_tree(rng, 9, 70, max_depth=3, roots=2)
    wl = W.make_workload("check", "bf16", parent, seg_len, H=8, Hkv=2, D=128, gH=2, dk=128, dv=128,
                         gates="sigmoid", root_state_std=None, seed=5)
    caps = caps_for(wl.parent, wl.seg_len, wl.H // wl.Hkv, kv_heads=wl.Hkv)
    sess = ForkSession(**caps, D=wl.D, gH=wl.gH, dk=wl.dk, dv=wl.dv)
    d = to_device(wl, "cuda")
    out = dict(o=torch.empty_like(d["q"]), lse=torch.empty((wl.T, wl.H), device="cuda"),
               go=torch.empty((wl.T, wl.gH, wl.dv), dtype=d["gq"].dtype, device="cuda"),
               s0=torch.empty((wl.S, wl.gH, wl.dv, wl.dk), device="cuda"))
    return wl, sess, d, out


def run(sess, d, out):
    for v in out.values():
        v.fill_(float("nan"))
    sess.attention(d["q"], d["k"], d["v"], out["o"], out["lse"])
    sess.gdn(d["gq"], d["gk"], d["gv"], d["a"], d["b"], out["go"], out["s0"])
    torch.cuda.synchronize()


def untouched(out):
    return all(bool(torch.isnan(v.float()).all()) for v in out.values())


def written(out):
    return all(bool(torch.isfinite(v.float()).all()) for v in out.values())


def test_clean_run_reports_no_device_error():
    wl, sess, d, out = setup()
    sess.build(wl.parent, wl.seg_len)
    run(sess, d, out)
    assert written(out)
    assert sess.check() == 0
    sess.close()


@pytest.mark.parametrize("word,value,bit", [(MH_MAGIC, 0, B.FORK_DEVERR_MAGIC),
                                            (MH_T, None, B.FORK_DEVERR_CAPACITY)])
def test_overwritten_header_stops_every_kernel(word, value, bit):
    wl, sess, d, out = setup()
    sess.build(wl.parent, wl.seg_len)
    if value is None:
        value = sess.caps.t_cap + 1  # a tree larger than the launch's capacity
    sess.blob.view(torch.int32)[word] = value
    run(sess, d, out)
    assert untouched(out), "a kernel wrote an output past a failed header check"
    with pytest.raises(B.ForkError) as e:
        sess.check()
    assert e.value.status == -7
    got = sess.check(raise_on_error=False)
    assert got == bit, got
    log(f"  header word {word} = {value}: device error word {got}, outputs untouched ({e.value})")
    # a new build clears the word, and the same launches run normally
    sess.build(wl.parent, wl.seg_len)
    run(sess, d, out)
    assert written(out)
    assert sess.check() == 0
    sess.close()


def test_graph_replay_on_a_blob_beyond_its_bucket_stops():
    """A graph recorded for one bucket, replayed after the blob's header was
    made to claim a larger tree: its kernels stop (their workspaces were
    sized for the bucket) and the word says so; rebuilt, it replays."""
    wl, sess, d, out = setup()
    sess.build(wl.parent, wl.seg_len)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sess.capture(dict(q=d["q"], k=d["k"], v=d["v"], o=out["o"], lse=out["lse"]),
                     dict(q=d["gq"], k=d["gk"], v=d["gv"], a=d["a"], b=d["b"], o=out["go"],
                          seg_start_state=out["s0"]))
    torch.cuda.synchronize()
    for v in out.values():
        v.fill_(float("nan"))
    sess.blob.view(torch.int32)[MH_T] = sess.caps.t_cap + 1
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        sess.replay()
    torch.cuda.synchronize()
    assert untouched(out)
    assert sess.check(stream=stream, raise_on_error=False) == B.FORK_DEVERR_CAPACITY
    with torch.cuda.stream(stream):
        sess.build(wl.parent, wl.seg_len)
        sess.replay()
    torch.cuda.synchronize()
    assert written(out)
    assert sess.check(stream=stream) == 0
    sess.close()
