"""Device buffers and calls of the hot path for one capacity bucket.

PyTorch provides device memory, pinned host memory and streams; every step of
the path runs in libforkattn.so through ``binding``. A ForkSession owns:

* the metadata blob (device) and a ring of pinned staging buffers, so a new
  tree can be planned on the host while the previous upload is still queued;
* the Gated DeltaNet workspace (sized for the bucket's capacities);
* optionally a recorded graph of both layers (``capture``).
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
FORK_DT = {"f32": B.FORK_F32, "bf16": B.FORK_BF16}


class ForkSession:
    """kv_heads and D (attention) enable split query tiles and size their
    workspace; gH, dk, dv (Gated DeltaNet) size the scan workspace."""

    def __init__(self, t_cap: int, s_cap: int, depth_cap: int, gqa_group: int,
                 kv_heads: int = 0, D: int = 0, gH: int = 0, dk: int = 0, dv: int = 0,
                 device: str = "cuda", ring: int = 2, ctx_cap: int = 0):
        self.caps = B.make_caps(t_cap, s_cap, depth_cap, gqa_group, kv_heads, ctx_cap)
        dev_bytes, stg_bytes = B.fork_meta_size(self.caps)
        self.device = torch.device(device)
        self.blob = torch.empty(dev_bytes, dtype=torch.uint8, device=self.device)
        self.staging = [torch.empty(stg_bytes, dtype=torch.uint8, pin_memory=True)
                        for _ in range(ring)]
        self.events = [None] * ring
        self._slot = 0
        self.meta = None
        self.gdn_ws = None
        self.attn_ws = None
        probe = B.fork_meta()
        probe.caps = self.caps
        if gH:
            n = B.gdn_fork_workspace(probe, gH, dk, dv, B.FORK_BF16)
            self.gdn_ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        if kv_heads and D:
            # sized for fp32 partials, the larger of the two dtypes
            n = B.fork_attn_workspace(probe, gqa_group * kv_heads, kv_heads, D, B.FORK_F32)
            if n:
                self.attn_ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        self.graph = None

    # -- metadata -----------------------------------------------------------
    def build(self, parent, seg_len, stream=None, ctx_start=None, ctx_len=None) -> B.fork_meta:
        """ctx_start / ctx_len: resumed contexts of the roots (cache rows), or None."""
        parent = np.ascontiguousarray(parent, np.int32)
        seg_len = np.ascontiguousarray(seg_len, np.int32)
        if ctx_len is not None:
            ctx_start = np.ascontiguousarray(ctx_start, np.int32)
            ctx_len = np.ascontiguousarray(ctx_len, np.int32)
        i = self._slot
        self._slot = (i + 1) % len(self.staging)
        if self.events[i] is not None:
            self.events[i].synchronize()  # the upload that last used this buffer is done
        self.meta = B.fork_meta_build_ctx(parent, seg_len, ctx_start, ctx_len, self.caps, self.blob,
                                          self.staging[i], stream=stream)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream() if stream is None else stream)
        self.events[i] = ev
        return self.meta

    def check(self, stream=None, raise_on_error: bool = True) -> int:
        """Device error word of the blob (synchronises the stream); raises
        ForkError (FORK_E_DEVICE) when a kernel stopped on the blob."""
        return B.fork_meta_check(self.meta, stream=stream, raise_on_error=raise_on_error)

    # -- layers -------------------------------------------------------------
    def attention(self, q, k, v, o, lse=None, scale: float = 0.0, stream=None, kc=None, vc=None):
        """kc / vc: key/value cache of resumed contexts [ctx_cap, Hkv, D] (required when the
        session has a context capacity)."""
        T, H, D = q.shape
        Hkv = k.shape[1]
        dt = B.FORK_BF16 if q.dtype == torch.bfloat16 else B.FORK_F32
        ws = self.attn_ws
        B.fork_attn_forward_ctx(self.meta, q, k, v, kc, vc, o, lse, H, Hkv, D, scale, dt, ws,
                                0 if ws is None else ws.numel(), stream=stream)

    def attention_qk8(self, q8, q_scale, k8, k_scale, v, o, lse=None, scale: float = 0.0, stream=None):
        """Tree attention with FP8 scores: q8 [T, H, D] / k8 [T, Hkv, D] E4M3 codes
        (uint8) with row scales q_scale [T, H] / k_scale [T, Hkv] (fork_quantize_fp8
        over rows of D), v bf16 [T, Hkv, D], o bf16 [T, H, D]."""
        T, H, D = q8.shape
        Hkv = k8.shape[1]
        ws = self.attn_ws
        B.fork_attn_forward_qk8(self.meta, q8, q_scale, k8, k_scale, v, o, lse, H, Hkv, D, scale, ws,
                                0 if ws is None else ws.numel(), stream=stream)

    def gdn(self, q, k, v, a, b, o, seg_start_state, seg_final_state=None, root_state=None,
            scale: float = 1.0, stream=None):
        T, H, dk = q.shape
        dv = v.shape[2]
        dt = B.FORK_BF16 if q.dtype == torch.bfloat16 else B.FORK_F32
        B.gdn_fork_forward(self.meta, q, k, v, a, b, root_state, o, seg_start_state,
                           seg_final_state, H, dk, dv, scale, dt, self.gdn_ws,
                           self.gdn_ws.numel(), stream=stream)

    def gdn_fp8(self, q8, q_scale, k8, k_scale, v8, v_scale, a, b, o, seg_start_state, seg_final_state=None,
                root_state=None, scale: float = 1.0, stream=None):
        """Gated DeltaNet with FP8 inputs: q8, k8, v8 [T, H, 128] E4M3 codes (uint8)
        with row scales [T, H] (fork_quantize_fp8 over rows of 128), o bf16."""
        T, H, dk = q8.shape
        B.gdn_fork_forward_fp8(self.meta, q8, q_scale, k8, k_scale, v8, v_scale, a, b, root_state, o,
                               seg_start_state, seg_final_state, H, dk, v8.shape[2], scale, stream=stream)

    # -- block pieces -------------------------------------------------------
    def rope(self, x, theta: float = 10000.0, stream=None):
        """Rotary embedding in place at the isolated positions; x [T, nheads, D]."""
        T, nh, D = x.shape
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_rope_forward(self.meta, x, nh, D, theta, dt, stream=stream)

    def conv(self, x, w, y, bias=None, conv_state=None, act: int = 1, stream=None):
        """Causal depthwise convolution along the isolated sequences; x, y [T, C],
        w [C, K] fp32, bias [C], conv_state [R, C, K-1]."""
        T, C = x.shape
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_conv_forward(self.meta, x, w, bias, conv_state, y, C, w.shape[1], act, dt, stream=stream)

    # -- mixer pieces -------------------------------------------------------
    def gate(self, x, g, w, y, mode: int, eps: float = 1e-6, stream=None, ld_g: int = 0):
        """Gate / norm over the last axis of x [T, nheads, D] (mode 0 x sigmoid(g),
        1 rmsnorm(x) w silu(g), 2 rmsnorm(x) w). g: a tensor [T, nheads, D], or with
        ld_g a device address whose token rows are ld_g elements apart."""
        T, nh, D = x.shape
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_gate_forward(self.meta, x, g, w, y, nh, D, mode, eps, dt, stream=stream, ld_g=ld_g)

    def option_readout(self, x, w, score=None, prob=None, stream=None):
        """Per-option scores and per-decision-group probabilities of the built
        tree from a layer's output x [T, ...] (rows of C = x[0].numel() values) and a
        readout vector w [C] fp32: the options are the leaf segments, grouped by
        parent. Returns (score, prob), fp32 [S] on the device (0 for segments that
        are not options)."""
        S = int(self.meta.num_segments)
        C = x[0].numel()
        if score is None:
            score = torch.empty(S, dtype=torch.float32, device=x.device)
        if prob is None:
            prob = torch.empty(S, dtype=torch.float32, device=x.device)
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_option_readout(self.meta, x, w, C, score, prob, dt, stream=stream)
        return score, prob

    def gdn_inputs(self, c, ab, a_log, dt_bias, q, k, v, a, b, eps: float = 1e-6, stream=None,
                   ld_ab: int = 0):
        """Gated DeltaNet inputs from the convolved projections c [T, 2 H dk + H dv]
        and the decay / write-strength projections ab [T, 2 H] (or, with ld_ab, a
        device address whose token rows are ld_ab elements apart). c None: only a
        and b (q, k, v come from gdn_conv_inputs_forward)."""
        T, H, dk = q.shape
        dv = v.shape[2]
        dt = B.FORK_BF16 if q.dtype == torch.bfloat16 else B.FORK_F32
        B.gdn_inputs_forward(self.meta, c, ab, a_log, dt_bias, q, k, v, a, b, H, dk, dv, eps, dt,
                             stream=stream, ld_ab=ld_ab)

    @staticmethod
    def linear(x, w, y, stream=None, accumulate: bool = False):
        """y [M, N] = x [M, K] w [N, K]^T (accumulate: y += x w^T)."""
        M, K = x.shape
        N = w.shape[0]
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_linear_forward(x, w, y, M, N, K, int(accumulate), dt, stream=stream)

    # -- FP8 ----------------------------------------------------------------
    def quantize_fp8(self, x, q=None, scale=None, stream=None):
        """Row-wise E4M3 quantisation on the GPU of x [rows, K]: returns (codes uint8
        of x's shape, scales [rows] fp32 on the device)."""
        rows, K = x.shape
        if q is None:
            q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if scale is None or scale.numel() != rows:
            scale = torch.empty(rows, dtype=torch.float32, device=x.device)
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.fork_quantize_fp8(x, q, scale, rows, K, dt, stream=stream)
        return q, scale

    @staticmethod
    def linear_fp8(xq, x_scale, wq, w_scale, y, stream=None, accumulate: bool = False):
        """y [M, N] bf16 = (xq [M, K] wq [N, K]^T) scaled by x_scale [M] and w_scale [N]
        (E4M3 codes with row scales)."""
        M, K = xq.shape
        N = wq.shape[0]
        B.fork_linear_fp8_forward(xq, x_scale, wq, w_scale, y, M, N, K, int(accumulate), stream=stream)

    def quantize_weights(self, W: dict, stream=None) -> dict:
        """A copy of mixer weights W with every projection (2-D "w*" entry) replaced
        by its (codes, scale) pair: the weights of an FP8 mixer."""
        out = {}
        for n, v in W.items():
            if n.startswith("w") and isinstance(v, torch.Tensor) and v.dim() == 2:
                out[n] = self.quantize_fp8(v, stream=stream)
            else:
                out[n] = v
        return out

    def _proj(self, fp8, xin, name, W, y, stream, accumulate=False):
        """One projection of a mixer: bf16/fp32, or FP8 with xin = (codes, scale)."""
        if fp8:
            wq, ws = W[name]
            self.linear_fp8(xin[0], xin[1], wq, ws, y, stream, accumulate)
        else:
            self.linear(xin, W[name], y, stream, accumulate)

    def _proj_in(self, fp8, x, b, key, stream):
        if not fp8:
            return x
        if x.dtype != torch.bfloat16:
            raise ValueError("FP8 projections write bf16: the mixer's activations must be bf16")
        q = b.get(key + "_q")
        if q is None or q.shape != x.shape:
            q = None
        return self.quantize_fp8(x, q, b.get(key + "_s"), stream)

    def attention_mixer(self, x, W: dict, theta: float = 10000.0, stream=None, bufs: dict = None,
                        residual=None, fp8: bool = False):
        """Attention mixer of a hybrid block on the current tree: projections, rotary
        embedding at the isolated positions, tree attention, sigmoid output gate,
        output projection. x [T, dm]; W holds device tensors wq, wk, wv, wg, wo and
        the ints H, Hkv, D. Returns y [T, dm], or with residual [T, dm] adds y into it
        (inside the output projection) and returns it. bufs: optional dict reused
        across calls for the intermediates. fp8: W from quantize_weights; the
        projections' inputs are quantised per token on the GPU."""
        T, dm = x.shape
        H, Hkv, D = W["H"], W["Hkv"], W["D"]
        b = self._bufs(bufs, x, dict(q=(T, H, D), k=(T, Hkv, D), v=(T, Hkv, D), g=(T, H, D),
                                     o=(T, H, D), u=(T, H, D), y=(T, dm)))
        xin = self._proj_in(fp8, x, b, "x", stream)
        if "wqkvg" in W:
            # one product for q | k | v | g, then split into contiguous heads
            # (rotating q and k on the way)
            nf = 2 * H * D + 2 * Hkv * D
            if "f" not in b or tuple(b["f"].shape) != (T, nf):
                b["f"] = torch.empty((T, nf), dtype=x.dtype, device=x.device)
            self._proj(fp8, xin, "wqkvg", W, b["f"], stream)
            dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
            base, esz = b["f"].data_ptr(), b["f"].element_size()
            col = 0
            for n, nh, th in (("q", H, theta), ("k", Hkv, theta), ("v", Hkv, 0.0), ("g", H, 0.0)):
                B.fork_rope_copy_forward(self.meta, base + col * esz, nf, b[n], nh, D, th, dt, stream=stream)
                col += nh * D
        else:
            for n in ("q", "k", "v", "g"):
                self._proj(fp8, xin, "w" + n, W, b[n], stream)
            self.rope(b["q"], theta, stream)
            self.rope(b["k"], theta, stream)
        self.attention(b["q"], b["k"], b["v"], b["o"], stream=stream)
        self.gate(b["o"], b["g"], None, b["u"], 0, stream=stream)
        uin = self._proj_in(fp8, b["u"].view(T, H * D), b, "u", stream)
        if fp8:
            b["x_q"], b["x_s"], b["u_q"], b["u_s"] = xin[0], xin[1], uin[0], uin[1]
        out = b["y"] if residual is None else residual
        self._proj(fp8, uin, "wo", W, out, stream, accumulate=residual is not None)
        return out

    def gdn_mixer(self, x, W: dict, eps: float = 1e-6, stream=None, bufs: dict = None,
                  seg_start_state=None, residual=None, fp8: bool = False):
        """Gated DeltaNet mixer of a hybrid block on the current tree: projections,
        causal convolution along the isolated sequences (+ SiLU), normalised inputs and
        gates, forked Gated DeltaNet, gated RMS norm, output projection. x [T, dm]; W
        holds device tensors wqkv, wab, wz, wo, conv_w, a_log, dt_bias, norm_w and the
        ints H, dk, dv. Returns y [T, dm] (or residual + y in residual, as
        attention_mixer)."""
        T, dm = x.shape
        H, dk, dv = W["H"], W["dk"], W["dv"]
        C = 2 * H * dk + H * dv
        b = self._bufs(bufs, x, dict(p=(T, C), ab=(T, 2 * H), q=(T, H, dk), k=(T, H, dk),
                                     v=(T, H, dv), o=(T, H, dv), z=(T, H, dv), u=(T, H, dv),
                                     y=(T, dm)))
        for n, shape in (("a", (T, H)), ("b", (T, H))):
            if n not in b or b[n].shape != shape:
                b[n] = torch.empty(shape, dtype=torch.float32, device=x.device)
        S = int(self.meta.num_segments)
        st = seg_start_state
        if st is None:
            if "st" not in b or b["st"].shape[0] < S:
                b["st"] = torch.empty((S, H, dv, dk), dtype=torch.float32, device=x.device)
            st = b["st"]
        xin = self._proj_in(fp8, x, b, "x", stream)
        self._proj(fp8, xin, "wqkv", W, b["p"], stream)
        if "wzab" in W:
            # one product for the output gate and the decay / strength projections
            nz = (W["wzab"][0] if fp8 else W["wzab"]).shape[0]
            if "zab" not in b or tuple(b["zab"].shape) != (T, nz):
                b["zab"] = torch.empty((T, nz), dtype=x.dtype, device=x.device)
            self._proj(fp8, xin, "wzab", W, b["zab"], stream)
            z, ld_z = b["zab"].data_ptr(), nz
            ab, ld_ab = b["zab"].data_ptr() + H * dv * b["zab"].element_size(), nz
        else:
            self._proj(fp8, xin, "wab", W, b["ab"], stream)
            self._proj(fp8, xin, "wz", W, b["z"].view(T, H * dv), stream)
            z, ld_z, ab, ld_ab = b["z"], 0, b["ab"], 0
        # convolution + SiLU + L2-normalised q / k heads, written straight to q, k, v;
        # then the decay and write strength
        dt = B.FORK_BF16 if x.dtype == torch.bfloat16 else B.FORK_F32
        B.gdn_conv_inputs_forward(self.meta, b["p"], W["conv_w"], None, None, b["q"], b["k"], b["v"], H, dk, dv,
                                  W["conv_w"].shape[1], eps, dt, stream=stream)
        self.gdn_inputs(None, ab, W["a_log"], W["dt_bias"], b["q"], b["k"], b["v"], b["a"], b["b"], eps, stream,
                        ld_ab=ld_ab)
        self.gdn(b["q"], b["k"], b["v"], b["a"], b["b"], b["o"], st, scale=dk ** -0.5, stream=stream)
        self.gate(b["o"], z, W["norm_w"], b["u"], 1, eps, stream, ld_g=ld_z)
        uin = self._proj_in(fp8, b["u"].view(T, H * dv), b, "u", stream)
        if fp8:
            b["x_q"], b["x_s"], b["u_q"], b["u_s"] = xin[0], xin[1], uin[0], uin[1]
        out = b["y"] if residual is None else residual
        self._proj(fp8, uin, "wo", W, out, stream, accumulate=residual is not None)
        return out

    def stack(self, x, layers, final_norm, theta: float = 10000.0, eps: float = 1e-6,
              stream=None, bufs: dict = None, fp8: bool = False):
        """Pre-norm residual stack on the current tree, in place on x [T, dm]:
        x <- x + mixer(rmsnorm(x) w_l) for each (kind, weights, norm weight) in
        layers (kind "attn" or "gdn"; the add happens in the output projection),
        then returns h = rmsnorm(x) w_final. fp8: layers' weights from
        quantize_weights, projections in FP8."""
        T, dm = x.shape
        b = self._bufs(bufs, x, dict(hn=(T, 1, dm), h=(T, 1, dm)))
        b.setdefault("mixers", {})
        for i, (kind, W, nw) in enumerate(layers):
            mb = b["mixers"].setdefault(i, {})
            self.gate(x.view(T, 1, dm), None, nw, b["hn"], 2, eps, stream)
            if kind == "attn":
                self.attention_mixer(b["hn"].view(T, dm), W, theta, stream, mb, residual=x, fp8=fp8)
            else:
                self.gdn_mixer(b["hn"].view(T, dm), W, eps, stream, mb, residual=x, fp8=fp8)
        self.gate(x.view(T, 1, dm), None, final_norm, b["h"], 2, eps, stream)
        return b["h"].view(T, dm)

    @staticmethod
    def fuse_attention_weights(W: dict) -> dict:
        """A copy of attention-mixer weights with wq | wk | wv | wg stacked into one
        [(2 H + 2 Hkv) D, dm] projection "wqkvg": attention_mixer then runs one product
        instead of four. (Row scales of FP8 weights are per output channel, so the
        stacked matrix quantises to the same codes.)"""
        out = dict(W)
        out["wqkvg"] = torch.cat([W["wq"], W["wk"], W["wv"], W["wg"]], dim=0).contiguous()
        return out

    @staticmethod
    def fuse_gdn_weights(W: dict) -> dict:
        """A copy of Gated DeltaNet mixer weights with wz | wab stacked into one
        [H dv + 2 H, dm] projection "wzab": gdn_mixer then runs one product for the
        output gate and the decay / strength inputs (the 2 H-wide product alone
        costs about as much as the H dv-wide one). Zero rows pad it to a multiple of
        8 outputs, so that each token's gate row stays 16-byte aligned."""
        out = dict(W)
        n = W["wz"].shape[0] + W["wab"].shape[0]
        pad = (-n) % 8
        parts = [W["wz"], W["wab"]]
        if pad:
            parts.append(torch.zeros((pad, W["wz"].shape[1]), dtype=W["wz"].dtype, device=W["wz"].device))
        out["wzab"] = torch.cat(parts, dim=0).contiguous()
        return out

    @staticmethod
    def _bufs(bufs, x, shapes):
        b = {} if bufs is None else bufs
        for n, shape in shapes.items():
            if n not in b or tuple(b[n].shape) != tuple(shape):
                b[n] = torch.empty(shape, dtype=x.dtype, device=x.device)
        return b

    # -- graphs -------------------------------------------------------------
    def capture(self, attn: dict, gdn: dict, stream=None) -> int:
        """Record both layers for this bucket. attn: q, k, v, o, lse, scale (and kc, vc
        when the bucket has a context capacity);
        gdn: q, k, v, a, b, root_state, o, seg_start_state, seg_final_state, scale.
        Tensors must be sized for the bucket capacity."""
        A = B.fork_graph_args()
        p = B._ptr
        A.q, A.k, A.v, A.o = p(attn["q"]), p(attn["k"]), p(attn["v"]), p(attn["o"])
        A.lse = p(attn.get("lse"))
        A.H, A.Hkv, A.D = attn["q"].shape[1], attn["k"].shape[1], attn["q"].shape[2]
        A.scale = float(attn.get("scale", 0.0))
        A.attn_ws = p(self.attn_ws)
        A.attn_ws_bytes = 0 if self.attn_ws is None else self.attn_ws.numel()
        A.gq, A.gk, A.gv = p(gdn["q"]), p(gdn["k"]), p(gdn["v"])
        A.a, A.b = p(gdn["a"]), p(gdn["b"])
        A.root_state = p(gdn.get("root_state"))
        A.go = p(gdn["o"])
        A.seg_start_state = p(gdn["seg_start_state"])
        A.seg_final_state = p(gdn.get("seg_final_state"))
        A.gH, A.dk, A.dv = gdn["q"].shape[1], gdn["q"].shape[2], gdn["v"].shape[2]
        A.gscale = float(gdn.get("scale", 1.0))
        A.gdn_ws, A.gdn_ws_bytes = p(self.gdn_ws), self.gdn_ws.numel()
        A.dt = B.FORK_BF16 if attn["q"].dtype == torch.bfloat16 else B.FORK_F32
        A.kc, A.vc = p(attn.get("kc")), p(attn.get("vc"))
        if self.graph is not None:
            B.fork_graph_destroy(self.graph)
        self.graph = B.fork_graph_create(self.meta, A, stream=stream)
        return self.graph

    def replay(self, stream=None):
        B.fork_graph_launch(self.graph, stream=stream)

    def close(self):
        if self.graph is not None:
            B.fork_graph_destroy(self.graph)
            self.graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# Capacity buckets of recorded graphs (tokens x segments; depth capacity 3):
# a compact set of fixed shapes that every request mix is padded into.
BUCKETS_T = [1 << 16, 1 << 17, 1 << 18, 3 << 17, 1 << 19]
BUCKETS_S = [1 << 9, 1 << 12, 1 << 13]
BUCKETS_DEPTH = [1, 3]  # a prefix with its options; deeper histories


def pick_depth_cap(depth: int) -> int:
    """The smallest depth bucket that holds a tree of this depth (a graph
    records one scan launch per depth level up to its cap, so shallow trees
    get a shallow bucket)."""
    for d in BUCKETS_DEPTH:
        if depth <= d:
            return d
    return int(depth)


def pick_bucket(T: int, S: int):
    """The smallest bucket (t_cap, s_cap) that holds T tokens and S segments."""
    for tc in BUCKETS_T:
        for sc in BUCKETS_S:
            if T <= tc and S <= sc:
                return tc, sc
    return int(T), int(S)


def caps_for(parent, seg_len, gqa_group: int, t_cap=None, s_cap=None, depth_cap=None,
             kv_heads: int = 0, ctx_cap: int = 0):
    """Exact capacities of one tree (eager use)."""
    parent = np.asarray(parent)
    depth = np.zeros(len(parent), np.int64)
    for s in range(len(parent)):
        if parent[s] >= 0:
            depth[s] = depth[parent[s]] + 1
    return dict(t_cap=t_cap or int(np.sum(seg_len)), s_cap=s_cap or len(parent),
                depth_cap=depth_cap if depth_cap is not None else int(depth.max()),
                gqa_group=gqa_group, kv_heads=kv_heads, ctx_cap=ctx_cap)


def to_device(wl, device="cuda"):
    """Device tensors of a workload (q/k/v in its dtype, a/b/root fp32)."""
    dt = TORCH_DT[wl.dtype]
    t = lambda x, d=dt: torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=d)
    out = dict(q=t(wl.q), k=t(wl.k), v=t(wl.v), gq=t(wl.gq), gk=t(wl.gk), gv=t(wl.gv),
               a=t(wl.a, torch.float32), b=t(wl.b, torch.float32))
    out["root_state"] = None if wl.root_state is None else t(wl.root_state, torch.float32)
    return out


def request_mix_to_device(seed: int, t_cap: int = 0, device="cuda", threads: int = 8,
                          n_requests: int = 64, out: dict = None):
    """The request mix of PCG64 seed `seed` (workloads.request_mix: tree and
    readout from the seed, each request's tensors from its own child stream)
    drawn request by request on the host (a thread pool draws ahead) and
    copied into device tensors of t_cap rows (at least T; rows past T are
    zero). out: existing tensors (e.g. a recorded graph's) to fill instead.
    Returns (parent, seg_len, tensors, readout vectors); the host never holds
    more than a few requests' values."""
    import concurrent.futures as cf

    from . import workloads as W

    rng = np.random.Generator(np.random.PCG64(seed))
    parent, seg_len = W.request_mix_tree(rng, n_requests)
    w = (W._normal(rng, (16 * 128,)), W._normal(rng, (16 * 128,)))
    T = int(np.sum(seg_len))
    n = max(T, int(t_cap))
    bf = torch.bfloat16
    z = lambda *s, d=bf: torch.zeros(*s, dtype=d, device=device)
    if out is None:
        out = dict(q=z(n, 16, 128), k=z(n, 2, 128), v=z(n, 2, 128), gq=z(n, 16, 128), gk=z(n, 16, 128),
                   gv=z(n, 16, 128), a=z(n, 16, d=torch.float32), b=z(n, 16, d=torch.float32),
                   root_state=None)
    else:
        for name in ("q", "k", "v", "gq", "gk", "gv", "a", "b"):
            assert out[name].shape[0] >= T, f"{name} holds {out[name].shape[0]} rows < T = {T}"
            out[name][T:].zero_()
    spans = W.request_spans(parent, seg_len)
    window = 2 * max(1, threads)  # requests drawn ahead of the copies
    with cf.ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        draw = lambda r: ex.submit(W.request_mix_request, seed, r, parent, seg_len, n_requests)
        futs = [draw(r) for r in range(min(window, len(spans)))]
        for r, (a, b, t0, t1) in enumerate(spans):
            wl = futs[r].result()
            futs[r] = None
            if r + window < len(spans):
                futs.append(draw(r + window))
            d = to_device(wl, device)
            for name in ("q", "k", "v", "gq", "gk", "gv", "a", "b"):
                out[name][t0:t1].copy_(d[name])
            del wl, d
    return parent, seg_len, out, w
