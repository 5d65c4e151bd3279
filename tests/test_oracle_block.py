"""Pins of the oracle's fork-aware block pieces (CPU): the rotary embedding at
isolated positions and the causal depthwise convolution along isolated
sequences, each checked against a different formulation (complex rotation,
numpy.convolve over the explicitly built isolated sequence) and against the
properties that define it."""
import numpy as np
import pytest

import oracle
from tests import brute


def path_tokens(parent, seg_len, s):
    """Token ids of s's isolated sequence (ancestors root first, then s)."""
    st = brute.seg_starts(seg_len)
    segs = list(reversed(brute.ancestors(parent, s))) + [s]
    return np.concatenate([np.arange(st[x], st[x] + seg_len[x]) for x in segs])


def rope_complex(x, pos, theta):
    """Rotation as complex multiplication: (x_i + i x_{i+D/2}) e^{i pos theta^(-2i/D)}."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    ang = np.asarray(pos, np.float64)[:, None, None] * theta ** (-2.0 * np.arange(D // 2) / D)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_single_segment_is_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 3, 16)).astype(np.float32)
    y = oracle.rope([-1], [37], x, theta=500.0)
    np.testing.assert_allclose(y, rope_complex(x, np.arange(37), 500.0), rtol=0, atol=1e-12)
    # a rotation: norms kept
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x.astype(np.float64), axis=-1),
                               rtol=1e-12)


def test_rope_scores_depend_on_offset_only():
    """<rope(q, m), rope(k, j)> for one fixed q and k depends on m - j only."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal(32).astype(np.float32)
    k = rng.standard_normal(32).astype(np.float32)
    n = 20
    yq = oracle.rope([-1], [n], np.tile(q, (n, 1, 1)))[:, 0]
    yk = oracle.rope([-1], [n], np.tile(k, (n, 1, 1)))[:, 0]
    G = yq @ yk.T
    for d in range(-n + 1, n):
        diag = np.diagonal(G, offset=d)
        np.testing.assert_allclose(diag, diag[0], rtol=0, atol=1e-10)


@pytest.mark.parametrize("seed", [3, 4])
def test_rope_tree_positions_are_isolated_positions(seed):
    """Every token of a tree (with resumed contexts) is rotated as in its
    isolated sequence: context length + ancestors' tokens + own position."""
    rng = np.random.default_rng(seed)
    from tree_structured_decision_amd import workloads as W
    parent, seg_len = W.random_tree(rng, 9, 12, max_depth=4, roots=2)
    ctx_len = np.where(parent < 0, rng.integers(0, 30, len(parent)), 0).astype(np.int32)
    T = int(seg_len.sum())
    x = rng.standard_normal((T, 2, 8)).astype(np.float32)
    y = oracle.rope(parent, seg_len, x, theta=10000.0, ctx_len=ctx_len)
    st = brute.seg_starts(seg_len)
    for s in range(len(parent)):
        toks = path_tokens(parent, seg_len, s)
        root = s
        while parent[root] >= 0:
            root = parent[root]
        pos = ctx_len[root] + np.arange(len(toks))
        own = slice(len(toks) - seg_len[s], len(toks))
        want = rope_complex(x[toks[own]], pos[own], 10000.0)
        np.testing.assert_allclose(y[st[s]:st[s] + seg_len[s]], want, rtol=0, atol=1e-10)


def conv_np(seq, w, bias, act, state=None):
    """numpy.convolve per channel over one explicit sequence [N, C] (state:
    K-1 earlier inputs, oldest first); 'full' mode truncated to causal."""
    seq = np.asarray(seq, np.float64)
    C, K = w.shape
    if state is not None:
        seq = np.concatenate([np.asarray(state, np.float64).T, seq])
    out = np.stack([np.convolve(seq[:, c], np.asarray(w[c], np.float64)[::-1])[:len(seq)]
                    for c in range(C)], axis=1)
    if bias is not None:
        out = out + np.asarray(bias, np.float64)
    if act:
        out = out / (1 + np.exp(-out))
    return out[K - 1:] if state is not None else out


@pytest.mark.parametrize("act", [0, 1])
def test_conv_single_segment_is_numpy_convolve(act):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((23, 6)).astype(np.float32)
    w = rng.standard_normal((6, 4)).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    y = oracle.conv([-1], [23], x, w, bias=b, act=act)
    np.testing.assert_allclose(y, conv_np(x, w, b, act), rtol=0, atol=1e-12)


def test_conv_tree_windows_fork_from_the_parent_tail():
    """Each segment's outputs equal numpy.convolve over its isolated sequence;
    segments shorter than the window reach back into grandparents."""
    rng = np.random.default_rng(6)
    parent = np.array([-1, 0, 1, 1, 0, 4, -1, 6], np.int32)
    seg_len = np.array([7, 1, 2, 5, 3, 1, 2, 4], np.int32)
    T, C, K = int(seg_len.sum()), 5, 4
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = rng.standard_normal((C, K)).astype(np.float32)
    y = oracle.conv(parent, seg_len, x, w, act=1)
    st = brute.seg_starts(seg_len)
    for s in range(len(parent)):
        toks = path_tokens(parent, seg_len, s)
        want = conv_np(x[toks], w, None, 1)[-seg_len[s]:]
        np.testing.assert_allclose(y[st[s]:st[s] + seg_len[s]], want, rtol=0, atol=1e-12)


def test_conv_state_continues_a_resumed_sequence():
    """With the last K-1 inputs of a resumed context as conv_state, a root's
    outputs equal the convolution of the context followed by its tokens."""
    rng = np.random.default_rng(7)
    C, K = 4, 4
    prefix = rng.standard_normal((9, C)).astype(np.float32)
    x = rng.standard_normal((6, C)).astype(np.float32)
    w = rng.standard_normal((C, K)).astype(np.float32)
    state = prefix[-(K - 1):].T[None].copy()  # [R=1, C, K-1], oldest first
    y = oracle.conv([-1], [6], x, w, conv_state=state, act=0)
    want = conv_np(np.concatenate([prefix, x]), w, None, 0)[-6:]
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-12)
