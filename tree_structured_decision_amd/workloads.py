"""Seeded synthetic inputs for the tree-flattened decision stream.

This module only draws random numbers and lays them out; it holds none of the
attention or Gated DeltaNet arithmetic. Both the HIP path and the CPU oracle
consume what it returns.

Tree and stream conventions (Flide page on kongchang.com, section
"ForkAttention: exact forking in GPU indices"): a decision request is a tree of
segments flattened into one token stream. Segment ``s`` has ``seg_len[s]``
tokens and parent ``parent[s]`` (``-1`` for a root, otherwise ``< s``);
segments are laid out contiguously in index order, so parents come before
children.

Draw order, fixed for every workload: tree, attention q, k, v, Gated DeltaNet
q, k, v, a, b, root state, readout vector. Every value is drawn in float32 with
``numpy.random.Generator(PCG64(seed))``; bf16 workloads are then rounded to
bf16 (round to nearest, ties to even) and kept as float32 arrays holding
exactly representable bf16 values. The Gated DeltaNet key is L2-normalised in
float32 before that rounding. ``a`` and ``b`` stay float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Seed of workload n (1-based, in the order of WORKLOADS below) is 1000 + n.
SEED_BASE = 1000


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("round_bf16 takes finite values")
    # finite floats have bit patterns <= 0xFF7FFFFF, so adding at most 0x8000
    # stays below 2^32 in uint32 arithmetic
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": q/k/v/o element type
    parent: np.ndarray              # int32 [S]
    seg_len: np.ndarray             # int32 [S]
    # softmax attention layer
    H: int
    Hkv: int
    D: int
    q: np.ndarray                   # [T, H, D]   float32 (bf16-exact for bf16)
    k: np.ndarray                   # [T, Hkv, D]
    v: np.ndarray                   # [T, Hkv, D]
    # Gated DeltaNet layer
    gH: int
    dk: int
    dv: int
    gq: np.ndarray                  # [T, gH, dk]
    gk: np.ndarray                  # [T, gH, dk]  (L2-normalised rows)
    gv: np.ndarray                  # [T, gH, dv]
    a: np.ndarray                   # [T, gH] float32 decay
    b: np.ndarray                   # [T, gH] float32 write strength
    root_state: Optional[np.ndarray]  # [R, gH, dv, dk] float32 or None (zero)
    w_attn: np.ndarray              # readout vector, [H*D]
    w_gdn: np.ndarray               # readout vector, [gH*dv]
    description: str = ""

    @property
    def T(self) -> int:
        return int(self.seg_len.sum())

    @property
    def S(self) -> int:
        return int(self.parent.shape[0])

    @property
    def R(self) -> int:
        return int((self.parent < 0).sum())


# --------------------------------------------------------------------------
# trees

def tree_one_level(prefix: int, option_lens) -> tuple[np.ndarray, np.ndarray]:
    """A root prefix followed by option segments that are all its children."""
    option_lens = [int(x) for x in option_lens]
    parent = np.array([-1] + [0] * len(option_lens), dtype=np.int32)
    seg_len = np.array([prefix] + option_lens, dtype=np.int32)
    return parent, seg_len


def tree_three_level(prefix: int, n_children: int, child_len: int,
                     n_options: int, option_len: int):
    """Root, then its children, then every child's options, breadth-first
    with siblings contiguous."""
    parent = [-1] + [0] * n_children
    seg_len = [prefix] + [child_len] * n_children
    for c in range(n_children):
        parent += [1 + c] * n_options
        seg_len += [option_len] * n_options
    return np.array(parent, np.int32), np.array(seg_len, np.int32)


def tree_requests(prefixes, option_lens_per_request):
    """Several independent requests, request-major: root r, then its options."""
    parent, seg_len = [], []
    for p, opts in zip(prefixes, option_lens_per_request):
        r = len(parent)
        parent.append(-1)
        seg_len.append(int(p))
        for L in opts:
            parent.append(r)
            seg_len.append(int(L))
    return np.array(parent, np.int32), np.array(seg_len, np.int32)


def reciprocal_int(rng: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    """n draws from P(x) proportional to 1/x on the inclusive integers [lo, hi]
    (the discrete reading of "log-uniform over integers")."""
    xs = np.arange(lo, hi + 1, dtype=np.float64)
    p = 1.0 / xs
    p /= p.sum()
    return rng.choice(np.arange(lo, hi + 1), size=n, p=p).astype(np.int64)


# --------------------------------------------------------------------------
# value draws

def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _sigmoid32(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_workload(name: str, dtype: str, parent, seg_len, *, H, Hkv, D, gH, dk, dv,
                  gates: str, root_state_std: Optional[float], seed: int,
                  rng: Optional[np.random.Generator] = None,
                  description: str = "", readout: bool = True) -> Workload:
    """Draw every tensor of a workload for a given tree.

    gates == "uniform": a ~ U(0.9, 1), b ~ U(0, 1).
    gates == "sigmoid": a = sigmoid(N(3, 0.5)), b = sigmoid(N(0, 1)).
    readout: draw the readout vectors last (False: leave them None).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    parent = np.asarray(parent, np.int32)
    seg_len = np.asarray(seg_len, np.int32)
    T = int(seg_len.sum())
    R = int((parent < 0).sum())
    q = _normal(rng, (T, H, D))
    k = _normal(rng, (T, Hkv, D))
    v = _normal(rng, (T, Hkv, D))
    gq = _normal(rng, (T, gH, dk))
    gk = _l2_rows(_normal(rng, (T, gH, dk)))
    gv = _normal(rng, (T, gH, dv))
    if gates == "uniform":
        a = rng.uniform(0.9, 1.0, size=(T, gH)).astype(np.float32)
        b = rng.uniform(0.0, 1.0, size=(T, gH)).astype(np.float32)
    elif gates == "sigmoid":
        a = _sigmoid32(rng.normal(3.0, 0.5, size=(T, gH)))
        b = _sigmoid32(rng.normal(0.0, 1.0, size=(T, gH)))
    else:
        raise ValueError(gates)
    root_state = None
    if root_state_std is not None:
        root_state = (rng.standard_normal(size=(R, gH, dv, dk), dtype=np.float32)
                      * np.float32(root_state_std)).astype(np.float32)
    w_attn = _normal(rng, (H * D,)) if readout else None
    w_gdn = _normal(rng, (gH * dv,)) if readout else None
    if dtype == "bf16":
        q, k, v, gq, gk, gv = (round_bf16(x) for x in (q, k, v, gq, gk, gv))
    elif dtype != "f32":
        raise ValueError(dtype)
    return Workload(name=name, dtype=dtype, parent=parent, seg_len=seg_len,
                    H=H, Hkv=Hkv, D=D, q=q, k=k, v=v, gH=gH, dk=dk, dv=dv,
                    gq=gq, gk=gk, gv=gv, a=a, b=b, root_state=root_state,
                    w_attn=w_attn, w_gdn=w_gdn, description=description)


# --------------------------------------------------------------------------
# the five decision workloads

def tiny_one_level(seed: int = SEED_BASE + 1) -> Workload:
    """Prefix 32 + 4 options of 8 tokens (64 tokens), fp32; attention 2 heads,
    D 64; Gated DeltaNet 2 heads, dk = dv = 32; uniform gates."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = tree_one_level(32, [8] * 4)
    return make_workload("tiny_one_level", "f32", parent, seg_len, H=2, Hkv=2, D=64,
                         gH=2, dk=32, dv=32, gates="uniform", root_state_std=None,
                         seed=seed, rng=rng,
                         description="prefix 32 + 4x8 options, fp32, attn 2/2/64, GDN 2x32x32")


def one_request(seed: int = SEED_BASE + 2) -> Workload:
    """Prefix 2048 + 16 options of U{16..48} tokens, bf16; attention 16/2/128;
    Gated DeltaNet 16 heads, dk = dv = 128; sigmoid gates."""
    rng = np.random.Generator(np.random.PCG64(seed))
    opts = rng.integers(16, 48, size=16, endpoint=True)
    parent, seg_len = tree_one_level(2048, opts)
    return make_workload("one_request", "bf16", parent, seg_len, H=16, Hkv=2, D=128,
                         gH=16, dk=128, dv=128, gates="sigmoid", root_state_std=None,
                         seed=seed, rng=rng,
                         description="prefix 2048 + 16 options of 16-48 tokens, bf16, "
                                     "attn 16/2/128, GDN 16x128x128")


def wide_options(seed: int = SEED_BASE + 3) -> Workload:
    """Prefix 8192 + 256 options of 8 tokens, bf16; attention 32/4/128 then
    Gated DeltaNet 16 heads, dk = dv = 128; uniform gates."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = tree_one_level(8192, [8] * 256)
    return make_workload("wide_options", "bf16", parent, seg_len, H=32, Hkv=4, D=128,
                         gH=16, dk=128, dv=128, gates="uniform", root_state_std=None,
                         seed=seed, rng=rng,
                         description="prefix 8192 + 256x8 options, bf16, attn 32/4/128, "
                                     "GDN 16x128x128")


def agent_history(seed: int = SEED_BASE + 4) -> Workload:
    """Prefix 4096, 8 children of 512, each with 32 options of 24 tokens, bf16;
    shapes as one_request; root state drawn from N(0, 0.1^2)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = tree_three_level(4096, 8, 512, 32, 24)
    return make_workload("agent_history", "bf16", parent, seg_len, H=16, Hkv=2, D=128,
                         gH=16, dk=128, dv=128, gates="sigmoid", root_state_std=0.1,
                         seed=seed, rng=rng,
                         description="prefix 4096 -> 8x512 children -> 32x24 options each, "
                                     "bf16, attn 16/2/128, GDN 16x128x128, root state N(0,0.1)")


def request_mix_tree(rng: np.random.Generator, n_requests: int = 64):
    prefixes = reciprocal_int(rng, 256, 16384, n_requests)
    counts = reciprocal_int(rng, 2, 256, n_requests)
    option_lens = [rng.integers(4, 32, size=int(c), endpoint=True) for c in counts]
    return tree_requests(prefixes, option_lens)


def request_spans(parent, seg_len):
    """(first segment, end segment, first token, end token) of every request of
    a request-major forest (a root followed by its subtree)."""
    parent = np.asarray(parent)
    seg_len = np.asarray(seg_len, np.int64)
    roots = np.flatnonzero(parent < 0)
    seg_end = np.append(roots[1:], len(parent))
    tok = np.concatenate([[0], np.cumsum(seg_len)])
    return [(int(a), int(b), int(tok[a]), int(tok[b])) for a, b in zip(roots, seg_end)]


def request_mix_request(seed: int, r: int, parent, seg_len, n_requests: int = 64,
                        w=None) -> Workload:
    """Request r of the request mix alone (its root re-indexed to segment 0):
    its q, k, v, Gated DeltaNet q, k, v, a, b come from the r-th child stream
    of SeedSequence(seed), in that order, so that one request's inputs can be
    drawn without the others'. w: the mix's readout vectors (w_attn, w_gdn)."""
    a, b, _, _ = request_spans(parent, seg_len)[r]
    p = np.asarray(parent[a:b], np.int32)
    p = np.where(p >= 0, p - a, -1).astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(n_requests)[r]))
    wl = make_workload(f"request_mix[{r}]", "bf16", p, np.asarray(seg_len[a:b], np.int32), H=16, Hkv=2,
                       D=128, gH=16, dk=128, dv=128, gates="sigmoid", root_state_std=None, seed=seed,
                       rng=rng, readout=False)
    if w is not None:
        wl.w_attn, wl.w_gdn = w
    return wl


def request_mix(seed: int = SEED_BASE + 5, n_requests: int = 64, select=None) -> Workload:
    """64 requests flattened into one stream, bf16: prefix lengths 1/P on
    256..16384, option counts 1/n on 2..256, option lengths U{4..32};
    shapes as one_request; zero root states. Draws: the tree and the readout
    vectors from PCG64(seed); each request's tensors from its own child
    stream (request_mix_request). select: request indices to keep (their
    sub-forest, in order), or None for the whole mix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = request_mix_tree(rng, n_requests)
    w = (_normal(rng, (16 * 128,)), _normal(rng, (16 * 128,)))
    rs = range(n_requests) if select is None else list(select)
    parts = [request_mix_request(seed, r, parent, seg_len, n_requests, w) for r in rs]
    par, sl = [], []
    for wl in parts:
        par.append(np.where(wl.parent >= 0, wl.parent + sum(len(x) for x in sl), -1))
        sl.append(wl.seg_len)
    cat = lambda n: np.concatenate([getattr(wl, n) for wl in parts])
    return Workload(name="request_mix", dtype="bf16", parent=np.concatenate(par).astype(np.int32),
                    seg_len=np.concatenate(sl).astype(np.int32), H=16, Hkv=2, D=128, q=cat("q"),
                    k=cat("k"), v=cat("v"), gH=16, dk=128, dv=128, gq=cat("gq"), gk=cat("gk"),
                    gv=cat("gv"), a=cat("a"), b=cat("b"), root_state=None, w_attn=w[0], w_gdn=w[1],
                    description="64 requests: prefixes 1/P on 256-16384, options 1/n on 2-256 of "
                                "U{4..32} tokens, bf16, attn 16/2/128, GDN 16x128x128")


WORKLOADS = {
    "tiny_one_level": tiny_one_level,
    "one_request": one_request,
    "wide_options": wide_options,
    "agent_history": agent_history,
    "request_mix": request_mix,
}


def random_tree(rng: np.random.Generator, n_segments: int, max_len: int,
                max_depth: int = 4, roots: int = 1):
    """A random valid tree with parents before children (used for small
    property tests). The first ``roots`` segments are roots."""
    parent = np.full(n_segments, -1, np.int32)
    depth = np.zeros(n_segments, np.int32)
    for s in range(roots, n_segments):
        cands = [p for p in range(s) if depth[p] < max_depth - 1]
        p = int(rng.choice(cands))
        parent[s] = p
        depth[s] = depth[p] + 1
    seg_len = rng.integers(1, max_len, size=n_segments, endpoint=True).astype(np.int32)
    return parent, seg_len


def group_options(parent: np.ndarray, seg_len: np.ndarray):
    """Decision groups: the leaf segments that share one parent, in index order.
    Returns a list of (parent, [leaf segments])."""
    parent = np.asarray(parent)
    S = parent.shape[0]
    has_child = np.zeros(S, bool)
    for s in range(S):
        if parent[s] >= 0:
            has_child[parent[s]] = True
    groups = {}
    for s in range(S):
        if not has_child[s] and parent[s] >= 0:
            groups.setdefault(int(parent[s]), []).append(s)
    return sorted(groups.items())


# --------------------------------------------------------------------------
# hybrid block weights (random init, no trained values)

def mixer_weights(seed: int, dm: int, *, H: int, Hkv: int, D: int, gH: int, dk: int, dv: int,
                  conv_k: int = 4, dtype: str = "bf16") -> dict:
    """Random weights of one attention mixer and one Gated DeltaNet mixer of
    model width dm. Projections are [out, in] with N(0, 1/in) entries (rounded
    to bf16 for bf16 runs); the convolution taps [C, conv_k] are N(0, 1/conv_k);
    a_log = log U(1, 16) and dt_bias = log(expm1(dt)) with dt log-uniform in
    [1e-3, 1e-1] (the usual decay initialisation); the output norm weight is
    1 + N(0, 0.1^2). Draw order: attention wq, wk, wv, wg, wo, then the
    Gated DeltaNet wqkv, wab, wz, wo, conv taps, a_log, dt_bias, norm weight."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def proj(n_out, n_in):
        w = _normal(rng, (n_out, n_in)) * np.float32(1.0 / np.sqrt(n_in))
        return round_bf16(w) if dtype == "bf16" else w.astype(np.float32)

    attn = dict(wq=proj(H * D, dm), wk=proj(Hkv * D, dm), wv=proj(Hkv * D, dm),
                wg=proj(H * D, dm), wo=proj(dm, H * D), H=H, Hkv=Hkv, D=D)
    C = 2 * gH * dk + gH * dv
    gdn = dict(wqkv=proj(C, dm), wab=proj(2 * gH, dm), wz=proj(gH * dv, dm), wo=proj(dm, gH * dv))
    gdn["conv_w"] = (_normal(rng, (C, conv_k)) * np.float32(1.0 / np.sqrt(conv_k))).astype(np.float32)
    gdn["a_log"] = np.log(rng.uniform(1.0, 16.0, size=gH)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=gH))
    gdn["dt_bias"] = np.log(np.expm1(dt)).astype(np.float32)
    gdn["norm_w"] = (1.0 + 0.1 * _normal(rng, (dv,))).astype(np.float32)
    gdn.update(H=gH, dk=dk, dv=dv)
    return {"attn": attn, "gdn": gdn}


def mixer_input(seed: int, T: int, dm: int, dtype: str = "bf16") -> np.ndarray:
    """Token activations x [T, dm] ~ N(0, 1) (bf16-rounded for bf16 runs)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (T, dm))
    return round_bf16(x) if dtype == "bf16" else x


def stack_weights(seed: int, dm: int, kinds=("gdn", "attn", "gdn", "attn"), *, H: int, Hkv: int, D: int,
                  gH: int, dk: int, dv: int, conv_k: int = 4, dtype: str = "bf16"):
    """Weights of a pre-norm residual stack of mixers: for each layer
    (kind, mixer weights, pre-norm weight [dm]); then the final norm weight
    [dm] and the option readout vector w_head [dm] ~ N(0, 1). Norm weights are
    1 + N(0, 0.1^2). Layer l's mixer weights come from mixer_weights(seed + 1 + l)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    layers = []
    for i, kind in enumerate(kinds):
        mw = mixer_weights(seed + 1 + i, dm, H=H, Hkv=Hkv, D=D, gH=gH, dk=dk, dv=dv, conv_k=conv_k, dtype=dtype)
        nw = (1.0 + 0.1 * _normal(rng, (dm,))).astype(np.float32)
        layers.append((kind, mw[kind], nw))
    final_norm = (1.0 + 0.1 * _normal(rng, (dm,))).astype(np.float32)
    w_head = _normal(rng, (dm,))
    return layers, final_norm, w_head
