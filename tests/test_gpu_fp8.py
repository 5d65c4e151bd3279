"""GPU parity of the FP8 (E4M3) pieces against the oracle, through the C ABI:
row-wise quantisation (codes and scales bit-exact: both sides decide them in
fp32 with correctly rounded divisions and nearest-even conversion), FP8
projections on the matrix cores, and the FP8 mixers and stack.

Tolerances:
* quantisation: codes and scales identical;
* FP8 projection: |gpu - oracle| <= 2^-8 |oracle| + 2^-14 (|xd| |wd|^T) on the
  decoded operands (the bf16 rounding of the output plus fp32 accumulation);
* FP8 mixers and stack against the oracle quantising at the same points with
  bf16-rounded intermediates: relative RMS error <= 3e-2 and max error <=
  1e-1 of the largest output (an intermediate that differs by one bf16
  rounding can move its fp8 code by one step, 2^-4 relative), and the options'
  softmax within TVD 2e-2."""
import numpy as np
import pytest
import torch

from oracle import mixer as OM
from tests.gpu_helpers import log
from tests.test_gpu_mixer import dev, dev_stack, host, session, to_dev_weights
from tree_structured_decision_amd import metrics
from tree_structured_decision_amd import workloads as W
from tree_structured_decision_amd.session import ForkSession

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,rows,K,scale", [("bf16", 2559, 2048, 1.0), ("f32", 37, 520, 300.0),
                                                ("bf16", 5, 8, 1e-3), ("f32", 64, 128, 1e-30)])
def test_quantize_fp8_bit_exact(dtype, rows, K, scale):
    rng = np.random.default_rng(rows + K)
    x = (rng.standard_normal((rows, K)) * rng.uniform(0.1, 3, (rows, 1)) * scale).astype(np.float32)
    x[rows // 2] = 0.0  # an all-zero row (scale 1)
    x[0, :4] = [448.0 * scale, -1e-8 * scale, 0.0, 2.0 ** -9 * scale]
    if dtype == "bf16":
        x = W.round_bf16(x)
    sess = ForkSession(t_cap=8, s_cap=1, depth_cap=0, gqa_group=1)
    q, s = sess.quantize_fp8(dev(x, dtype))
    torch.cuda.synchronize()
    rq, rs = OM.quantize_fp8(x)
    qg, sg = q.cpu().numpy(), s.cpu().numpy()
    bad = int((qg != rq).sum())
    log(f"  quantize {dtype} {rows}x{K}: {bad} codes differ, scales equal: {np.array_equal(sg, rs)}")
    assert np.array_equal(sg, rs)
    assert bad == 0


@pytest.mark.parametrize("M,N,K,acc", [(300, 72, 256, False), (2559, 2048, 2048, False), (129, 40, 96, True)])
def test_linear_fp8_parity(M, N, K, acc):
    rng = np.random.default_rng(M)
    x = W.round_bf16(rng.standard_normal((M, K)).astype(np.float32))
    w = W.round_bf16((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    y0 = W.round_bf16(rng.standard_normal((M, N)).astype(np.float32))
    sess = ForkSession(t_cap=8, s_cap=1, depth_cap=0, gqa_group=1)
    xq, xs = sess.quantize_fp8(dev(x, "bf16"))
    wq, ws = sess.quantize_fp8(dev(w, "bf16"))
    y = dev(y0, "bf16") if acc else torch.full((M, N), float("nan"), device="cuda", dtype=torch.bfloat16)
    sess.linear_fp8(xq, xs, wq, ws, y, accumulate=acc)
    torch.cuda.synchronize()
    rqx, rsx = OM.quantize_fp8(x)
    rqw, rsw = OM.quantize_fp8(w)
    ref = OM.linear_fp8(rqx, rsx, rqw, rsw) + (y0 if acc else 0.0)
    bound = np.abs(OM.dequantize_fp8(rqx, rsx)) @ np.abs(OM.dequantize_fp8(rqw, rsw)).T
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * bound
    err = np.abs(host(y) - ref)
    log(f"  linear fp8 {M}x{N}x{K} acc={acc}: max err {err.max():.3e}, max err / tol {(err / tol).max():.3f}")
    assert np.isfinite(err).all() and (err <= tol).all()


def compare_fp8(name, got, ref):
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max() / np.abs(ref).max()
    log(f"  {name}: relative RMS error {rel:.3e}, max error / max |y| {mx:.3e}")
    assert np.isfinite(got).all() and rel <= 3e-2 and mx <= 1e-1, name


def test_fp8_mixers_and_stack_one_request():
    wl = W.one_request()
    heads = dict(H=16, Hkv=2, D=128, gH=16, dk=128, dv=128)
    sess = session(wl.parent, wl.seg_len, group=8, kv_heads=2, D=128, gH=16, dk=128, dv=128)
    Wt = W.mixer_weights(81, 2048, **heads)
    x = W.mixer_input(82, wl.T, 2048)
    xd = dev(x, "bf16")
    A = sess.quantize_weights(ForkSession.fuse_attention_weights(to_dev_weights(Wt["attn"], "bf16")))
    G = sess.quantize_weights(ForkSession.fuse_gdn_weights(to_dev_weights(Wt["gdn"], "bf16")))
    ya = host(sess.attention_mixer(xd, A, fp8=True))
    yg = host(sess.gdn_mixer(xd, G, fp8=True))
    compare_fp8("fp8 attention mixer", ya, OM.attention_mixer(wl.parent, wl.seg_len, x, Wt["attn"], bf16=True, fp8=True))
    compare_fp8("fp8 GDN mixer", yg, OM.gdn_mixer(wl.parent, wl.seg_len, x, Wt["gdn"], bf16=True, fp8=True))

    layers, fn, w_head = W.stack_weights(83, 2048, **heads)
    dl, dfn = dev_stack(layers, fn, "bf16")
    dl = [(k, sess.quantize_weights(Wl), nw) for k, Wl, nw in dl]
    xs = W.mixer_input(84, wl.T, 2048)
    h = host(sess.stack(dev(xs, "bf16"), dl, dfn, fp8=True))
    ref = OM.stack(wl.parent, wl.seg_len, xs, layers, fn, bf16=True, fp8=True)
    compare_fp8("fp8 stack of 4", h, ref)
    fid = metrics.decision_fidelity(h, ref, w_head, wl.parent, wl.seg_len)
    log(f"  option distributions vs the fp8 oracle: {fid}")
    assert fid["tvd_max"] <= 2e-2
