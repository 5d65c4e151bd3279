"""Brute-force fp64 references over the flattened token stream (test helper).

These compute the same quantities as the oracle by a different route: one
dense [T, T] tree mask over the whole stream for attention, and a token-level
recurrence whose predecessor is the previous token of the segment, or the
parent segment's last token at a segment start, for the Gated DeltaNet. The
pages claim that the tree-flattened evaluation equals isolated per-branch
forward passes (kongchang.com page, section "ForkAttention: exact forking in
GPU indices"); checking the isolated-path oracle against this stream-level
brute force is that claim made executable. Tiny trees only.
"""
import numpy as np


def seg_starts(seg_len):
    seg_len = np.asarray(seg_len, np.int64)
    return np.concatenate([[0], np.cumsum(seg_len)[:-1]])


def ancestors(parent, s):
    out = []
    p = int(parent[s])
    while p >= 0:
        out.append(p)
        p = int(parent[p])
    return out


def brute_mask(parent, seg_len):
    """M[t, j] = token j's segment is an ancestor of t's segment, or is t's own
    segment with j <= t."""
    st = seg_starts(seg_len)
    T = int(np.sum(seg_len))
    tok_seg = np.repeat(np.arange(len(seg_len)), seg_len)
    M = np.zeros((T, T), bool)
    for t in range(T):
        s = tok_seg[t]
        anc = set(ancestors(parent, s))
        for j in range(T):
            sj = tok_seg[j]
            M[t, j] = (sj in anc) or (sj == s and j <= t)
    return M


def brute_attention(parent, seg_len, q, k, v, scale=None):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    M = brute_mask(parent, seg_len)
    o = np.zeros((T, H, D))
    lse = np.zeros((T, H))
    for h in range(H):
        z = scale * (q[:, h] @ k[:, h // G].T)
        z = np.where(M, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        l = p.sum(axis=1, keepdims=True)
        o[:, h] = (p @ v[:, h // G]) / l
        lse[:, h] = (m + np.log(l))[:, 0]
    return o, lse


def brute_gdn(parent, seg_len, q, k, v, a, b, root_state=None, scale=1.0):
    """Token-level recurrence over the stream. Returns (o, start, final)."""
    q, k, v, a, b = (np.asarray(x, np.float64) for x in (q, k, v, a, b))
    T, H, dk = q.shape
    dv = v.shape[2]
    S = len(seg_len)
    st = seg_starts(seg_len)
    roots = [s for s in range(S) if parent[s] < 0]
    after = np.zeros((T, H, dv, dk))
    o = np.zeros((T, H, dv))
    start = np.zeros((S, H, dv, dk))
    final = np.zeros((S, H, dv, dk))
    for s in range(S):
        if parent[s] >= 0:
            p = int(parent[s])
            prev = after[st[p] + seg_len[p] - 1]
        elif root_state is not None:
            prev = np.asarray(root_state[roots.index(s)], np.float64)
        else:
            prev = np.zeros((H, dv, dk))
        start[s] = prev
        for i in range(int(seg_len[s])):
            t = st[s] + i
            for h in range(H):
                Sm = prev[h]
                kk = k[t, h]
                I = np.eye(dk)
                Sn = a[t, h] * Sm @ (I - b[t, h] * np.outer(kk, kk)) + b[t, h] * np.outer(v[t, h], kk)
                after[t, h] = Sn
                o[t, h] = scale * Sn @ q[t, h]
            prev = after[t]
        final[s] = after[st[s] + seg_len[s] - 1]
    return o, start, final
