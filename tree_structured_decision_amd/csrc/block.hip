// Fork-aware pieces of a hybrid block around the attention and Gated DeltaNet
// layers. Every branch must evaluate exactly as its isolated forward pass
// (Flide, kongchang.com page, section "ForkAttention: exact forking in GPU
// indices"), so an operation that reads a token's position or its
// predecessors reads them in the token's isolated sequence, through the same
// GPU-resident segment metadata:
//   - rotary position embedding at tok_iso_pos (resumed context, ancestors'
//     tokens and own position counted);
//   - the short causal depthwise convolution of a Gated DeltaNet block, whose
//     window at a segment's first tokens continues into the parent's tail
//     (further ancestors for short parents) and, before a root, into the
//     root's saved convolution state.
// Both are streaming kernels bound by HBM: one read and one write of the
// activations (the convolution's earlier taps are cache hits), coalesced in
// 16-byte vectors along the channel dimension.
#include <math.h>

#include "common.h"

namespace fork {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f(unsigned short u) { return __uint_as_float((unsigned)u << 16); }
__device__ __forceinline__ unsigned short f_to_bf16(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }

// ---------------------------------------------------------------- rotary
// A thread rotates 4 pairs (i, i + D/2), i = 4 k .. 4 k + 3, of one (token,
// head). The angle pos * theta^(-2i/D) is formed and reduced modulo 2 pi in
// double precision (positions reach 10^5..10^6, where a float angle would
// be off by ~0.01 rad), then its sine and cosine are taken in float.
constexpr int kRopeThreads = 256;
constexpr int kMaxRopeD = 256;

// The rows are read from src (row stride ld_src elements per token, head h
// at column h D) and written to dst [T, nh, D] contiguous; src == dst with
// ld_src = nh D rotates in place. rotate = false copies (the split of a fused
// projection's output into contiguous heads).
template <bool BF16>
__global__ void __launch_bounds__(kRopeThreads) rope_kernel(const int32_t* __restrict__ blob, const void* src,
                                                            long long ld_src, void* dst, int nh, int D,
                                                            double log2_theta, int rotate, BlobGuard guard) {
  __shared__ double inv_freq[kMaxRopeD / 2];
  if (!blob_ok(blob, guard)) return;
  const int half = D / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) inv_freq[i] = exp2(-(2.0 * i / D) * log2_theta);
  __syncthreads();
  const int T = blob[MH_T];
  const int32_t* __restrict__ iso = blob + blob[MH_OFF_TOKISO];
  const int per_row = half / 4;  // threads per (token, head)
  const long long n = (long long)T * nh * per_row;
  const double two_pi = 6.283185307179586476925286766559;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int k = (int)(idx % per_row);
    const long long th = idx / per_row;  // token * nh + head
    const int t = (int)(th / nh), h = (int)(th % nh);
    float c[4] = {1.f, 1.f, 1.f, 1.f}, s[4] = {0.f, 0.f, 0.f, 0.f};
    if (rotate) {
      const double pos = (double)iso[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        double a = pos * inv_freq[4 * k + e];
        a -= two_pi * rint(a / two_pi);
        sincosf((float)a, &s[e], &c[e]);
      }
    }
    const long long so = (long long)t * ld_src + (long long)h * D;
    if constexpr (BF16) {
      const unsigned short* in = (const unsigned short*)src + so;
      unsigned short* row = (unsigned short*)dst + th * D;
      const u32x2_t lo = *(const u32x2_t*)(in + 4 * k);
      const u32x2_t hi = *(const u32x2_t*)(in + half + 4 * k);
      float a0[4] = {bf16_to_f(lo.x & 0xffff), bf16_to_f(lo.x >> 16), bf16_to_f(lo.y & 0xffff), bf16_to_f(lo.y >> 16)};
      float b0[4] = {bf16_to_f(hi.x & 0xffff), bf16_to_f(hi.x >> 16), bf16_to_f(hi.y & 0xffff), bf16_to_f(hi.y >> 16)};
      unsigned short ra[4], rb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ra[e] = f_to_bf16(a0[e] * c[e] - b0[e] * s[e]);
        rb[e] = f_to_bf16(b0[e] * c[e] + a0[e] * s[e]);
      }
      *(u32x2_t*)(row + 4 * k) = u32x2_t{ra[0] | ((unsigned)ra[1] << 16), ra[2] | ((unsigned)ra[3] << 16)};
      *(u32x2_t*)(row + half + 4 * k) = u32x2_t{rb[0] | ((unsigned)rb[1] << 16), rb[2] | ((unsigned)rb[3] << 16)};
    } else {
      const float* in = (const float*)src + so;
      float* row = (float*)dst + th * D;
      const f32x4_t a0 = *(const f32x4_t*)(in + 4 * k);
      const f32x4_t b0 = *(const f32x4_t*)(in + half + 4 * k);
      f32x4_t ra, rb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ra[e] = a0[e] * c[e] - b0[e] * s[e];
        rb[e] = b0[e] * c[e] + a0[e] * s[e];
      }
      *(f32x4_t*)(row + 4 * k) = ra;
      *(f32x4_t*)(row + half + 4 * k) = rb;
    }
  }
}

// ------------------------------------------------------------ convolution
// A thread computes 8 consecutive channels of a run of kConvRun consecutive
// tokens, with the channels' taps and a sliding window of the last K inputs
// in registers, so every input row and weight is read once per run. Inside a
// segment the window shifts by one token; at a segment's first K - 1 tokens
// (and at the run's first token) it is refilled by walking back through the
// segment metadata: within the segment, then into the parent's last tokens
// (repeatedly, for parents shorter than the window); before a root's first
// token the root's convolution state supplies the inputs (or zeros).
constexpr int kConvThreads = 256;

// Gated DeltaNet input split (SPLIT = true): channels [0, Cq) are the query
// heads, [Cq, 2 Cq) the key heads, the rest the value heads, each head G * 8
// channels wide; query and key heads are L2-normalised after the activation,
// x / sqrt(|x|^2 + eps), and the three parts go to separate [T, heads, dk]
// arrays. The G lanes holding one head's channels for a token run are
// consecutive and aligned (the per-token channel groups are a multiple of
// G), and all follow the same run, so the norm is a G-lane shuffle sum.
struct ConvSplit {
  void* yk;
  void* yv;
  int Cq;
  int G;
  float eps;
};

template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ base, long long off, float* v) {
  if constexpr (BF16) {
    const u32x4_t p = *(const u32x4_t*)((const unsigned short*)base + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f(p[e] & 0xffff);
      v[2 * e + 1] = bf16_to_f(p[e] >> 16);
    }
  } else {
    const f32x4_t a = *(const f32x4_t*)((const float*)base + off);
    const f32x4_t b = *(const f32x4_t*)((const float*)base + off + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

constexpr int kConvRun = 8;

template <bool BF16, int K, bool SPLIT>
__global__ void __launch_bounds__(kConvThreads) conv_kernel(const int32_t* __restrict__ blob,
                                                            const void* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            const float* __restrict__ state,
                                                            void* __restrict__ y, int C, int act, ConvSplit sp,
                                                            BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const int T = blob[MH_T];
  const int32_t* __restrict__ tok_seg = blob + blob[MH_OFF_TOKSEG];
  const int32_t* __restrict__ tok_pos = blob + blob[MH_OFF_TOKPOS];
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ root_ord = blob + blob[MH_OFF_ROOTORD];
  const int per_tok = C / 8;
  const long long n = (long long)((T + kConvRun - 1) / kConvRun) * per_tok;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (long long)gridDim.x * blockDim.x) {
    const int run = (int)(idx / per_tok);
    const int c0 = 8 * (int)(idx - (long long)run * per_tok);
    const int t0 = run * kConvRun, t1 = min(T, t0 + kConvRun);
    // the 8 channels' taps: 8 K consecutive floats of w
    float wt[8 * K];
#pragma unroll
    for (int i = 0; i < 2 * K; ++i) {
      const f32x4_t v = *(const f32x4_t*)(w + (long long)c0 * K + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[4 * i + e] = v[e];
    }
    float b8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b8[e] = bias ? bias[c0 + e] : 0.f;
    float win[K][8];  // win[K-1-j]: the input j tokens back
    for (int t = t0; t < t1; ++t) {
      const int p = tok_pos[t];
      if (t > t0 && p > 0) {
        // same segment as t - 1: shift the window by one token
#pragma unroll
        for (int i = 0; i + 1 < K; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) win[i][e] = win[i + 1][e];
        load8<BF16>(x, (long long)t * C + c0, win[K - 1]);
      } else {
        const int s = tok_seg[t];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          float* v = win[K - 1 - j];
          if (p >= j) {
            load8<BF16>(x, (long long)(t - j) * C + c0, v);
            continue;
          }
          // position p - j of segment s, walked back into ancestors
          int cs = s, cp = p - j;
          while (cp < 0 && parent[cs] >= 0) {
            cs = parent[cs];
            cp += seg_len[cs];
          }
          if (cp >= 0) {
            load8<BF16>(x, (long long)(seg_start[cs] + cp) * C + c0, v);
          } else if (state && cp >= -(K - 1)) {
            // cs is the root: its state holds the K-1 inputs before its first token
            const float* st = state + ((long long)root_ord[cs] * C + c0) * (K - 1) + (K - 1) + cp;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = st[e * (K - 1)];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
          }
        }
      }
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] = b8[e];
#pragma unroll
        for (int i = 0; i < K; ++i) acc[e] += wt[e * K + i] * win[i][e];
      }
      if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] / (1.f + __expf(-acc[e]));
      }
      void* out = y;
      long long orow = (long long)t * C + c0;
      if constexpr (SPLIT) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += acc[e] * acc[e];
        for (int o = sp.G >> 1; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        const int region = c0 < sp.Cq ? 0 : (c0 < 2 * sp.Cq ? 1 : 2);
        if (region < 2) {
          const float r = 1.f / sqrtf(ss + sp.eps);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] *= r;
        }
        out = region == 0 ? y : (region == 1 ? sp.yk : sp.yv);
        orow = region == 2 ? (long long)t * (C - 2 * sp.Cq) + (c0 - 2 * sp.Cq)
                           : (long long)t * sp.Cq + (c0 - region * sp.Cq);
      }
      if constexpr (BF16) {
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f_to_bf16(acc[2 * e]) | ((unsigned)f_to_bf16(acc[2 * e + 1]) << 16);
        *(u32x4_t*)((unsigned short*)out + orow) = o;
      } else {
        float* o = (float*)out + orow;
        *(f32x4_t*)o = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *(f32x4_t*)(o + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
      }
    }
  }
}

int stream_grid(long long threads, int per_block) {
  const long long want = (threads + per_block - 1) / per_block;
  const long long cap = (long long)device_cu_count() * 16;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

fork_status launch_rope(const fork_meta* m, const void* src, long long ld_src, void* dst, int nh, int D, float theta,
                        fork_dtype dt, hipStream_t stream) {
  const long long threads = (long long)m->caps.t_cap * nh * (D / 8);
  const int grid = stream_grid(threads, kRopeThreads);
  const int rotate = theta > 0.f;
  const double l2t = rotate ? log2((double)theta) : 0.0;
  if (dt == FORK_BF16)
    hipLaunchKernelGGL(rope_kernel<true>, dim3(grid), dim3(kRopeThreads), 0, stream, (const int32_t*)m->dev, src,
                       ld_src, dst, nh, D, l2t, rotate, blob_guard(m->caps));
  else
    hipLaunchKernelGGL(rope_kernel<false>, dim3(grid), dim3(kRopeThreads), 0, stream, (const int32_t*)m->dev, src,
                       ld_src, dst, nh, D, l2t, rotate, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

template <bool BF16, int K, bool SPLIT>
fork_status launch_conv_k(const fork_meta* m, const void* x, const float* w, const float* bias, const float* state,
                          void* y, int C, int act, ConvSplit sp, hipStream_t stream) {
  const long long threads = (long long)((m->caps.t_cap + kConvRun - 1) / kConvRun) * (C / 8);
  const int grid = stream_grid(threads, kConvThreads);
  hipLaunchKernelGGL((conv_kernel<BF16, K, SPLIT>), dim3(grid), dim3(kConvThreads), 0, stream, (const int32_t*)m->dev,
                     x, w, bias, state, y, C, act, sp, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

template <bool BF16, bool SPLIT>
fork_status launch_conv_t(const fork_meta* m, const void* x, const float* w, const float* bias, const float* state,
                          void* y, int C, int K, int act, ConvSplit sp, hipStream_t stream) {
  switch (K) {
    case 2: return launch_conv_k<BF16, 2, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    case 3: return launch_conv_k<BF16, 3, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    case 4: return launch_conv_k<BF16, 4, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    case 5: return launch_conv_k<BF16, 5, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    case 6: return launch_conv_k<BF16, 6, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    case 7: return launch_conv_k<BF16, 7, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
    default: return launch_conv_k<BF16, 8, SPLIT>(m, x, w, bias, state, y, C, act, sp, stream);
  }
}

fork_status launch_conv(const fork_meta* m, const void* x, const float* w, const float* bias, const float* state,
                        void* y, int C, int K, int act, fork_dtype dt, hipStream_t stream) {
  const ConvSplit none{nullptr, nullptr, 0, 1, 0.f};
  if (dt == FORK_BF16) return launch_conv_t<true, false>(m, x, w, bias, state, y, C, K, act, none, stream);
  return launch_conv_t<false, false>(m, x, w, bias, state, y, C, K, act, none, stream);
}

fork_status launch_conv_split(const fork_meta* m, const void* x, const float* w, const float* bias,
                              const float* state, void* q, void* k, void* v, int H, int dk, int dv, int K, float eps,
                              fork_dtype dt, hipStream_t stream) {
  const int C = 2 * H * dk + H * dv;
  const ConvSplit sp{k, v, H * dk, dk / 8, eps};
  if (dt == FORK_BF16) return launch_conv_t<true, true>(m, x, w, bias, state, q, C, K, 1, sp, stream);
  return launch_conv_t<false, true>(m, x, w, bias, state, q, C, K, 1, sp, stream);
}

}  // namespace fork
