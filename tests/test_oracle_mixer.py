"""Pins of the mixer oracle (oracle/mixer.py) against what mathematics fixes:
rounding ties, symmetries of sigmoid and softplus, the scale invariance of
the RMS norm, brute-force products, a one-token stream where attention and
the Gated DeltaNet have closed forms, and the exactness of forking
(kongchang.com page, section "ForkAttention: exact forking in GPU indices":
every branch equals its isolated forward pass)."""
import numpy as np
import pytest

from oracle import mixer as M
from tree_structured_decision_amd import workloads as W


def test_to_bf16_ties_and_bit_rounding():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1)
    assert M.to_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert M.to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert M.to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert M.to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7  # above the tie
    assert M.to_bf16(0.0) == 0.0
    # on float32 inputs it agrees with the bit-level rounding of the input module
    x = np.random.default_rng(0).standard_normal(20000).astype(np.float32) * 37.0
    assert np.array_equal(M.to_bf16(x.astype(np.float64)), W.round_bf16(x).astype(np.float64))


def test_linear_brute_force():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((5, 7)), rng.standard_normal((3, 7))
    y = M.linear(x, w)
    for i in range(5):
        for j in range(3):
            assert abs(y[i, j] - sum(x[i, t] * w[j, t] for t in range(7))) < 1e-12


def test_sigmoid_gate_symmetry():
    rng = np.random.default_rng(2)
    x, g = rng.standard_normal((6, 3, 16)), 3 * rng.standard_normal((6, 3, 16))
    # sigmoid(g) + sigmoid(-g) = 1
    assert np.allclose(M.gate(x, g, None, 0) + M.gate(x, -g, None, 0), x, atol=1e-14)
    assert np.allclose(M.gate(x, np.zeros_like(g), None, 0), x / 2, atol=1e-15)


def test_rms_norm_properties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, 64)) * 5
    w = 1.0 + 0.1 * rng.standard_normal(64)
    g = rng.standard_normal((4, 2, 64))
    one = np.ones(64)
    y = M.gate(x, None, one, 2, eps=1e-12)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-9)  # unit mean square
    assert np.allclose(M.gate(7.5 * x, None, w, 2, eps=1e-12), M.gate(x, None, w, 2, eps=1e-12), atol=1e-10)
    # eps enters as mean(x^2) + eps
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(M.gate(x, None, one, 2, eps=0.5) ** 2, axis=-1), ms / (ms + 0.5), atol=1e-12)
    # silu(g) - silu(-g) = g
    d = M.gate(x, g, w, 1, eps=1e-6) - M.gate(x, -g, w, 1, eps=1e-6)
    assert np.allclose(d, M.gate(x, None, w, 2, eps=1e-6) * g, atol=1e-12)


def test_gdn_inputs_properties():
    rng = np.random.default_rng(4)
    T, H, dk, dv = 9, 3, 16, 8
    c = rng.standard_normal((T, 2 * H * dk + H * dv)) * 2
    u = rng.standard_normal((T, H)) * 4
    beta = rng.standard_normal((T, H)) * 3
    a_log = np.log(rng.uniform(1, 16, H))
    zero = np.zeros(H)
    q, k, v, a, b = M.gdn_inputs(c, np.concatenate([u, beta], 1), a_log, zero, H, dk, dv, eps=1e-12)
    _, _, _, a_neg, b_neg = M.gdn_inputs(c, np.concatenate([-u, -beta], 1), a_log, zero, H, dk, dv, eps=1e-12)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-9)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-9)
    cq = c[:, :H * dk].reshape(T, H, dk)
    ck = c[:, H * dk:2 * H * dk].reshape(T, H, dk)
    assert np.allclose(q * np.linalg.norm(cq, axis=-1, keepdims=True), cq, atol=1e-9)  # direction kept
    assert np.allclose(k * np.linalg.norm(ck, axis=-1, keepdims=True), ck, atol=1e-9)
    assert np.array_equal(v, c[:, 2 * H * dk:].reshape(T, H, dv))
    # softplus(u) - softplus(-u) = u, so log a(u) - log a(-u) = -exp(a_log) u
    assert np.allclose(np.log(a) - np.log(a_neg), -np.exp(a_log) * u, atol=1e-10)
    assert np.allclose(b + b_neg, 1.0, atol=1e-14)
    assert ((a > 0) & (a < 1)).all()
    # dt_bias shifts the softplus argument
    _, _, _, a_b, _ = M.gdn_inputs(c, np.concatenate([u - 0.3, beta], 1), a_log, zero + 0.3, H, dk, dv)
    assert np.allclose(a_b, a, rtol=1e-12)
    # eps enters as |c|^2 + eps
    q1, _, _, _, _ = M.gdn_inputs(c, np.concatenate([u, beta], 1), a_log, zero, H, dk, dv, eps=2.0)
    n2 = np.sum(cq * cq, axis=-1)
    assert np.allclose(np.linalg.norm(q1, axis=-1) ** 2, n2 / (n2 + 2.0), atol=1e-12)


def small_weights(seed=5, dm=32):
    return W.mixer_weights(seed, dm, H=4, Hkv=2, D=16, gH=2, dk=16, dv=16, conv_k=4, dtype="f32")


def test_one_token_closed_forms():
    """One token, one segment: attention over a single key returns its value
    (for query head h the value of kv head h // (H / Hkv)), rotary position 0
    is the identity; the Gated DeltaNet from a zero state gives
    o = scale b (k . q) v, and the convolution sees only its last tap."""
    dm = 32
    Wt = small_weights(6, dm)
    x = W.mixer_input(7, 1, dm, "f32").astype(np.float64)
    parent, seg_len = np.array([-1], np.int32), np.array([1], np.int32)
    A = Wt["attn"]
    v = (x @ A["wv"].T).reshape(1, 2, 16)
    g = (x @ A["wg"].T).reshape(1, 4, 16)
    o = v[:, [0, 0, 1, 1], :]
    y_ref = ((o / (1 + np.exp(-g))).reshape(1, 64)) @ A["wo"].T
    y = M.attention_mixer(parent, seg_len, x, A)
    assert np.allclose(y, y_ref, rtol=1e-5, atol=1e-5)  # the layer oracle takes float32 inputs

    G = Wt["gdn"]
    H, dk, dv = 2, 16, 16
    p = x @ G["wqkv"].T
    c = p * G["conv_w"][:, -1][None, :]
    c = c / (1 + np.exp(-c))
    cq, ck = c[:, :H * dk].reshape(H, dk), c[:, H * dk:2 * H * dk].reshape(H, dk)
    cv = c[:, 2 * H * dk:].reshape(H, dv)
    qn = cq / np.sqrt((cq ** 2).sum(-1, keepdims=True) + 1e-6)
    kn = ck / np.sqrt((ck ** 2).sum(-1, keepdims=True) + 1e-6)
    beta = (x @ G["wab"].T)[0, H:]
    bb = 1 / (1 + np.exp(-beta))
    og = (bb * (kn * qn).sum(-1) / np.sqrt(dk))[:, None] * cv
    z = (x @ G["wz"].T).reshape(H, dv)
    u = og / np.sqrt((og ** 2).mean(-1, keepdims=True) + 1e-6) * G["norm_w"] * z / (1 + np.exp(-z))
    y_ref = u.reshape(1, H * dv) @ G["wo"].T
    y = M.gdn_mixer(parent, seg_len, x, G)
    assert np.allclose(y, y_ref, rtol=1e-4, atol=1e-5)


def path_segments(parent, s):
    p = []
    while s >= 0:
        p.append(s)
        s = parent[s]
    return p[::-1]


@pytest.mark.parametrize("seed", [11, 12])
def test_mixers_equal_isolated_paths(seed):
    """Each leaf's path through the tree, run as one isolated sequence, gives
    the same rows as the tree run (rotary positions, convolution windows that
    cross segment boundaries, attention visibility, forked states)."""
    rng = np.random.default_rng(seed)
    parent, seg_len = W.random_tree(rng, 9, 7, max_depth=4, roots=2)
    seg_len[rng.integers(0, 9, 3)] = 1  # windows reach past short parents
    T = int(seg_len.sum())
    dm = 32
    Wt = small_weights(seed, dm)
    x = W.mixer_input(seed + 1, T, dm, "f32").astype(np.float64)
    ya = M.attention_mixer(parent, seg_len, x, Wt["attn"])
    yg = M.gdn_mixer(parent, seg_len, x, Wt["gdn"])
    start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    leaves = [s for s in range(len(parent)) if not (parent == s).any()]
    for leaf in leaves:
        rows = np.concatenate([np.arange(start[s], start[s] + seg_len[s]) for s in path_segments(parent, leaf)])
        one = (np.array([-1], np.int32), np.array([len(rows)], np.int32))
        ia = M.attention_mixer(*one, x[rows], Wt["attn"])
        ig = M.gdn_mixer(*one, x[rows], Wt["gdn"])
        assert np.allclose(ya[rows], ia, rtol=1e-9, atol=1e-9)
        assert np.allclose(yg[rows], ig, rtol=1e-9, atol=1e-9)


def test_bf16_rounding_points_stay_close():
    """Rounding the stored intermediates to bf16 moves the mixers' outputs by
    about the bf16 resolution, not more."""
    rng = np.random.default_rng(13)
    parent, seg_len = W.random_tree(rng, 6, 12, max_depth=3)
    T = int(seg_len.sum())
    Wt = W.mixer_weights(14, 64, H=4, Hkv=2, D=16, gH=2, dk=16, dv=16, dtype="bf16")
    x = W.mixer_input(15, T, 64, "bf16").astype(np.float64)
    for f in (M.attention_mixer, M.gdn_mixer):
        key = "attn" if f is M.attention_mixer else "gdn"
        y64, y16 = f(parent, seg_len, x, Wt[key]), f(parent, seg_len, x, Wt[key], bf16=True)
        rel = np.linalg.norm(y16 - y64) / np.linalg.norm(y64)
        assert 1e-5 < rel < 2 ** -6, rel


def test_stack_with_silent_layers_is_the_final_norm():
    """With every output projection zero, the residual stream is never
    changed: the stack returns rmsnorm(x) w_final of the input."""
    rng = np.random.default_rng(16)
    parent, seg_len = W.random_tree(rng, 5, 6, max_depth=3)
    T = int(seg_len.sum())
    layers, fn, _ = W.stack_weights(17, 32, H=4, Hkv=2, D=16, gH=2, dk=16, dv=16, dtype="f32")
    silent = []
    for kind, Wl, nw in layers:
        Wl = dict(Wl)
        Wl["wo"] = np.zeros_like(Wl["wo"])
        silent.append((kind, Wl, nw))
    x = W.mixer_input(18, T, 32, "f32").astype(np.float64)
    h = M.stack(parent, seg_len, x, silent, fn)
    ref = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6) * fn
    assert np.allclose(h, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fp8", [False, True])
def test_stack_equals_isolated_paths(fp8):
    rng = np.random.default_rng(19)
    parent, seg_len = W.random_tree(rng, 8, 6, max_depth=4)
    seg_len[rng.integers(0, 8, 3)] = 1
    T = int(seg_len.sum())
    layers, fn, _ = W.stack_weights(20, 32, H=4, Hkv=2, D=16, gH=2, dk=16, dv=16, dtype="f32")
    x = W.mixer_input(21, T, 32, "f32").astype(np.float64)
    h = M.stack(parent, seg_len, x, layers, fn, fp8=fp8)
    start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    for leaf in [s for s in range(len(parent)) if not (parent == s).any()]:
        rows = np.concatenate([np.arange(start[s], start[s] + seg_len[s]) for s in path_segments(parent, leaf)])
        hi = M.stack(np.array([-1], np.int32), np.array([len(rows)], np.int32), x[rows], layers, fn, fp8=fp8)
        assert np.allclose(h[rows], hi, rtol=1e-9, atol=1e-9)


def test_e4m3_codes_from_the_format_definition():
    # every non-NaN code decodes and re-encodes to itself
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    v = M.e4m3_decode(codes)
    back = M.e4m3_encode(v)
    assert np.array_equal(back[np.abs(v) > 0], codes[np.abs(v) > 0])
    assert M.e4m3_decode(0x7E) == 448.0 and M.e4m3_decode(0x38) == 1.0 and M.e4m3_decode(0xB8) == -1.0
    assert M.e4m3_decode(0x01) == 2.0 ** -9 and M.e4m3_decode(0x08) == 2.0 ** -6
    assert np.isnan(M.e4m3_decode(0x7F))
    # values are strictly increasing over the positive codes
    pos = M.e4m3_decode(np.arange(0, 0x7F))
    assert (np.diff(pos) > 0).all()
    # ties go to the even mantissa: 1 + 1/16 between 1 and 1.125 -> 1; 1 + 3/16 -> 1.25
    assert M.e4m3_encode(1.0625) == 0x38 and M.e4m3_encode(1.1875) == 0x3A
    # a subnormal tie (2.5 * 2^-9) goes to 2 * 2^-9; the largest subnormal rounds up to 2^-6
    assert M.e4m3_encode(2.5 * 2.0 ** -9) == 0x02 and M.e4m3_encode(7.75 * 2.0 ** -9) == 0x08
    # carries into the next binade: 1.9375 is halfway between 1.875 and 2 -> 2 (even)
    assert M.e4m3_encode(1.9375) == 0x40
    # nearest: on random values the error is at most half a step
    x = np.random.default_rng(22).uniform(-448, 448, 5000)
    d = M.e4m3_decode(M.e4m3_encode(x))
    step = np.where(np.abs(x) >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.abs(x))).astype(int) - 3), 2.0 ** -9)
    assert (np.abs(d - x) <= step / 2 + 1e-12).all()


def test_quantize_fp8_row_scales_and_extremes():
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((6, 512)) * rng.uniform(0.01, 30, (6, 1))).astype(np.float32)
    q, s = M.quantize_fp8(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # each row's largest magnitude maps to +-448 (code 0x7E / 0xFE)
    assert ((q[np.arange(6), np.argmax(np.abs(x), axis=1)] & 0x7F) == 0x7E).all()
    # relative error of values in the normal range is at most 2^-4
    d = M.dequantize_fp8(q, s)
    big = np.abs(x) >= 2.0 ** -6 * s[:, None]
    assert (np.abs(d - x)[big] <= 2.0 ** -4 * np.abs(x)[big] * (1 + 1e-6)).all()
    # rows are independent: quantising one row alone gives the same codes
    q1, s1 = M.quantize_fp8(x[3:4])
    assert np.array_equal(q1[0], q[3]) and s1[0] == s[3]
    z, sz = M.quantize_fp8(np.zeros((2, 16), np.float32))
    assert (sz == 1.0).all() and (z == 0).all()
    # a product of quantised operands is the product of their decoded values
    w = rng.standard_normal((5, 64)).astype(np.float32)
    xx = rng.standard_normal((3, 64)).astype(np.float32)
    qx, sx = M.quantize_fp8(xx)
    qw, sw = M.quantize_fp8(w)
    assert np.allclose(M.linear_fp8(qx, sx, qw, sw), M.dequantize_fp8(qx, sx) @ M.dequantize_fp8(qw, sw).T, rtol=1e-12)


def test_fp8_mixers_equal_isolated_paths():
    """With per-token activation scales the FP8 mixers keep the isolated-pass
    equivalence: each leaf's path alone gives the tree's rows."""
    rng = np.random.default_rng(24)
    parent, seg_len = W.random_tree(rng, 7, 6, max_depth=3)
    T = int(seg_len.sum())
    Wt = small_weights(25, 32)
    x = W.mixer_input(26, T, 32, "f32").astype(np.float64)
    ya = M.attention_mixer(parent, seg_len, x, Wt["attn"], fp8=True)
    yg = M.gdn_mixer(parent, seg_len, x, Wt["gdn"], fp8=True)
    start = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
    for leaf in [s for s in range(len(parent)) if not (parent == s).any()]:
        rows = np.concatenate([np.arange(start[s], start[s] + seg_len[s]) for s in path_segments(parent, leaf)])
        one = (np.array([-1], np.int32), np.array([len(rows)], np.int32))
        assert np.allclose(ya[rows], M.attention_mixer(*one, x[rows], Wt["attn"], fp8=True), rtol=1e-9, atol=1e-9)
        assert np.allclose(yg[rows], M.gdn_mixer(*one, x[rows], Wt["gdn"], fp8=True), rtol=1e-9, atol=1e-9)


def _mutant_gate(x, g, w, mode, eps=1e-6):
    # silu replaced by sigmoid in the gated norm
    x = np.asarray(x, np.float64)
    if mode == 0:
        return x * M.sigmoid(g)
    r = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)
    return r * M.sigmoid(g) if mode == 1 else r


def _mutant_encode(t):
    # truncation instead of nearest-even rounding
    t = np.asarray(t, np.float64)
    a = np.abs(t)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = a >= 2.0 ** -6
    m = np.where(normal, np.floor((a / np.ldexp(1.0, e) - 1.0) * 8.0), np.floor(a / 2.0 ** -9)).astype(np.int64)
    ef = np.where(normal, e + 7, 0)
    return ((np.signbit(t).astype(np.int64) << 7) | (ef << 3) | m).astype(np.uint8)


@pytest.mark.parametrize("name,attr,mutant,pin", [
    ("silu -> sigmoid in the gated norm", "gate", _mutant_gate, "test_rms_norm_properties"),
    ("softplus sign flipped", "softplus", lambda x: np.logaddexp(0.0, -np.asarray(x, np.float64)),
     "test_gdn_inputs_properties"),
    ("bf16 ties away from zero", "to_bf16",
     lambda x: (lambda m, e: np.ldexp(np.sign(m) * np.floor(np.abs(m) * 256.0 + 0.5) / 256.0, e))(*np.frexp(np.asarray(x, np.float64))),
     "test_to_bf16_ties_and_bit_rounding"),
    ("e4m3 truncation", "e4m3_encode", _mutant_encode, "test_e4m3_codes_from_the_format_definition"),
    ("residual dropped", "_out", lambda r, u, wo, residual, fp8=False: r(M._lin(u, wo, fp8)),
     "test_stack_with_silent_layers_is_the_final_norm"),
])
def test_pins_catch_planted_mistakes(monkeypatch, name, attr, mutant, pin):
    """Each planted mistake in the mixer oracle makes a pin fail (the mistake
    is planted in the oracle, on the CPU)."""
    monkeypatch.setattr(M, attr, mutant)
    with pytest.raises(AssertionError):
        globals()[pin]()
