// Per-token pieces of the two token mixers of a hybrid block, on the
// flattened stream. None of them looks at other tokens, so a token of any
// branch is processed exactly as in its isolated forward pass (Flide,
// kongchang.com page, section "ForkAttention: exact forking in GPU indices")
// and the shared prefix is processed once:
//   - the output gate of the attention mixer, o * sigmoid(g);
//   - the gated RMS norm at the output of the Gated DeltaNet mixer,
//     rmsnorm(o) * w * silu(z), and the plain RMS norm in front of a mixer;
//   - the Gated DeltaNet inputs after the short convolution: L2-normalised
//     query and key heads, the value heads, and the per-head decay and
//     write strength from their projections;
//   - row-wise FP8 (E4M3) quantisation of the projections' operands.
// The pages describe the layers, not these surroundings; the forms follow the
// published Gated DeltaNet layer (Yang, Kautz, Hatamizadeh, "Gated Delta
// Networks", 2024) and sigmoid output gating of attention.
// All are streaming kernels bound by HBM: a group of L lanes (a power of two
// up to 64) owns one row of D elements and moves it in 16-byte vectors; the
// second read of a normalised row is a cache hit.
#include <math.h>

#include "common.h"

namespace fork {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMixThreads = 256;

__device__ __forceinline__ float bf16_to_f(unsigned short u) { return __uint_as_float((unsigned)u << 16); }
__device__ __forceinline__ unsigned short f_to_bf16(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }

// Elements i .. i + 7 of p (i a multiple of 8).
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, size_t i, float* v) {
  if constexpr (BF16) {
    const u32x4_t u = *(const u32x4_t*)((const unsigned short*)p + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(u[e] << 16);
      v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  } else {
    const f32x4_t a = *(const f32x4_t*)((const float*)p + i), b = *(const f32x4_t*)((const float*)p + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* p, size_t i, const float* v) {
  if constexpr (BF16) {
    u32x4_t u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (unsigned)f_to_bf16(v[2 * e]) | ((unsigned)f_to_bf16(v[2 * e + 1]) << 16);
    *(u32x4_t*)((unsigned short*)p + i) = u;
  } else {
    *(f32x4_t*)((float*)p + i) = f32x4_t{v[0], v[1], v[2], v[3]};
    *(f32x4_t*)((float*)p + i + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + expf(-x)); }

// Sum over the L lanes of a row group (groups are aligned runs of L lanes).
__device__ __forceinline__ float group_sum(float s, int L) {
  for (int o = L >> 1; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  return s;
}

// mode 0: y = x * sigmoid(g)
// mode 1: y = x / sqrt(mean(x^2) + eps) * w * silu(g)
// mode 2: y = x / sqrt(mean(x^2) + eps) * w
// over rows of D elements; T * nh rows, T read from the blob. g of token t,
// head h starts at g + t ldg + h D (ldg = nh D when g is [T, nh, D]).
template <bool BF16, int MODE>
__global__ void __launch_bounds__(kMixThreads) gate_kernel(const int32_t* __restrict__ blob, const void* x,
                                                           const void* g, long long ldg, const float* __restrict__ w,
                                                           void* y, int nh, int D, int L, float eps,
                                                           BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const long long rows = (long long)blob[MH_T] * nh;
  const int lane = threadIdx.x & 63, li = lane & (L - 1), rpw = 64 / L, nc = D / 8;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r0 = wave * rpw; r0 < rows; r0 += nwaves * rpw) {  // uniform over the wave
    const long long r = r0 + lane / L;
    const bool live = r < rows;
    const size_t base = (size_t)r * D;
    const size_t gbase = (size_t)(r / nh) * ldg + (size_t)(r % nh) * D;
    float scale = 1.f;
    if constexpr (MODE != 0) {
      float ss = 0.f;
      if (live)
        for (int j = li; j < nc; j += L) {
          float v[8];
          load8<BF16>(x, base + 8 * j, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        }
      ss = group_sum(ss, L);
      scale = 1.f / sqrtf(ss / (float)D + eps);
    }
    if (!live) continue;
    for (int j = li; j < nc; j += L) {
      float v[8], gv[8], o[8];
      load8<BF16>(x, base + 8 * j, v);
      if constexpr (MODE != 2) load8<BF16>(g, gbase + 8 * j, gv);
      if constexpr (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[e] * sigmoid(gv[e]);
      } else {
        const f32x4_t w0 = *(const f32x4_t*)(w + 8 * j), w1 = *(const f32x4_t*)(w + 8 * j + 4);
        const float ww[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = v[e] * scale * ww[e];
          if constexpr (MODE == 1) o[e] *= gv[e] * sigmoid(gv[e]);
        }
      }
      store8<BF16>(y, base + 8 * j, o);
    }
  }
}

// One (token, head) row per group of L lanes: c [T, 2 H dk + H dv] holds
// the convolved query, key and value heads side by side (null: the
// convolution already wrote q, k and v, only a and b are formed); ab the
// decay and write-strength projections of token t at ab + t ld_ab (2 H values).
template <bool BF16>
__global__ void __launch_bounds__(kMixThreads) gdn_inputs_kernel(
    const int32_t* __restrict__ blob, const void* c, const void* ab, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, void* q, void* k, void* v, float* __restrict__ a, float* __restrict__ b, int H,
    int dk, int dv, long long ld_ab, int L, float eps, BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const long long rows = (long long)blob[MH_T] * H;
  const int lane = threadIdx.x & 63, li = lane & (L - 1), rpw = 64 / L;
  const size_t cw = (size_t)2 * H * dk + (size_t)H * dv;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r0 = wave * rpw; r0 < rows; r0 += nwaves * rpw) {
    const long long r = r0 + lane / L;
    const bool live = r < rows;
    const long long t = r / H;
    const int h = (int)(r % H);
    const size_t cq = (size_t)t * cw + (size_t)h * dk, ck = cq + (size_t)H * dk,
                 cv = (size_t)t * cw + (size_t)2 * H * dk + (size_t)h * dv;
    float sq = 0.f, sk = 0.f;
    if (live && c)
      for (int j = li; j < dk / 8; j += L) {
        float vq[8], vk[8];
        load8<BF16>(c, cq + 8 * j, vq);
        load8<BF16>(c, ck + 8 * j, vk);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sq += vq[e] * vq[e];
          sk += vk[e] * vk[e];
        }
      }
    sq = group_sum(sq, L);
    sk = group_sum(sk, L);
    if (!live) continue;
    const float rq = 1.f / sqrtf(sq + eps), rk = 1.f / sqrtf(sk + eps);
    for (int j = li; c && j < dk / 8; j += L) {
      float vq[8], vk[8];
      load8<BF16>(c, cq + 8 * j, vq);
      load8<BF16>(c, ck + 8 * j, vk);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vq[e] *= rq;
        vk[e] *= rk;
      }
      store8<BF16>(q, (size_t)r * dk + 8 * j, vq);
      store8<BF16>(k, (size_t)r * dk + 8 * j, vk);
    }
    for (int j = li; c && j < dv / 8; j += L) {
      float vv[8];
      load8<BF16>(c, cv + 8 * j, vv);
      store8<BF16>(v, (size_t)r * dv + 8 * j, vv);
    }
    if (li == 0) {
      float al, be;
      if constexpr (BF16) {
        al = bf16_to_f(((const unsigned short*)ab)[(size_t)t * ld_ab + h]);
        be = bf16_to_f(((const unsigned short*)ab)[(size_t)t * ld_ab + H + h]);
      } else {
        al = ((const float*)ab)[(size_t)t * ld_ab + h];
        be = ((const float*)ab)[(size_t)t * ld_ab + H + h];
      }
      // softplus in the form that neither overflows nor cancels
      const float u = al + dt_bias[h];
      const float sp = fmaxf(u, 0.f) + log1pf(expf(-fabsf(u)));
      a[r] = expf(-expf(a_log[h]) * sp);
      b[r] = sigmoid(be);
    }
  }
}

// ------------------------------------------------------------ FP8 (E4M3)
// Row-wise quantisation to the OCP FP8 E4M3 format (bias 7, 3 mantissa bits,
// largest finite 448): for each row of K values, scale = amax / 448 (1 for an
// all-zero row) and code = RNE_e4m3(clamp(x / scale, -448, 448)), both
// divisions correctly rounded fp32, the conversion the hardware's
// nearest-even one. A row is one token (activations) or one output channel
// (weights), so a token's codes depend on that token alone: quantising the
// flattened stream gives every branch what its isolated pass would get.
template <bool BF16>
__global__ void __launch_bounds__(kMixThreads) quant_rows_kernel(const void* x, unsigned char* __restrict__ q,
                                                                 float* __restrict__ scales, long long rows, int K,
                                                                 int L) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63, li = lane & (L - 1), rpw = 64 / L, nc = K / 8;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r0 = wave * rpw; r0 < rows; r0 += nwaves * rpw) {  // uniform over the wave
    const long long r = r0 + lane / L;
    const bool live = r < rows;
    const size_t base = (size_t)r * K;
    float m = 0.f;
    if (live)
      for (int j = li; j < nc; j += L) {
        float v[8];
        load8<BF16>(x, base + 8 * j, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
      }
    for (int o = L >> 1; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (!live) continue;
    const float scale = m > 0.f ? m / 448.f : 1.f;
    if (li == 0) scales[r] = scale;
    for (int j = li; j < nc; j += L) {
      float v[8];
      load8<BF16>(x, base + 8 * j, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(v[e] / scale, -448.f), 448.f);
      unsigned lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
      unsigned hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
      *(u32x2_t*)(q + base + 8 * j) = u32x2_t{lo, hi};
    }
  }
}

// Lanes per row: the largest power of two <= min(64, D / 8).
int lanes_per_row(int D) {
  int L = 1;
  while (2 * L <= 64 && 2 * L <= D / 8) L *= 2;
  return L;
}

// Decision readout (a reading: the pages rank engines by the probabilities
// they give the options, kongchang.com page, section on performance, but
// define no scoring head). Options are the leaf segments; those sharing a
// parent form one decision group. Option c's score is <w, x[last token of c]>
// scaled by 1/sqrt(C), and its probability the softmax of the group's scores.
//
// Scores: one wave per segment (grid-stride); lane j sums the products of
// 8-element column groups j, j + 64, ..., then a butterfly sum. Every
// segment that is not an option gets score 0 and probability 0 here; the
// probabilities of options are written by readout_softmax_kernel.
template <bool BF16>
__global__ void __launch_bounds__(kMixThreads) readout_score_kernel(const int32_t* __restrict__ blob, const void* x,
                                                                    const float* __restrict__ w, int C,
                                                                    float inv_sqrt_c, float* __restrict__ score,
                                                                    float* __restrict__ prob, BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const int S = blob[MH_S];
  const int32_t* parent = blob + blob[MH_OFF_PARENT];
  const int32_t* first_child = blob + blob[MH_OFF_FIRSTCHILD];
  const int32_t* seg_start = blob + blob[MH_OFF_SEGSTART];
  const int32_t* seg_len = blob + blob[MH_OFF_SEGLEN];
  const int lane = threadIdx.x & 63, nc = C / 8;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  for (int s = wave; s < S; s += nwaves) {  // uniform over the wave
    const bool option = parent[s] >= 0 && first_child[s] < 0;
    float acc = 0.f;
    if (option) {
      const size_t base = (size_t)(seg_start[s] + seg_len[s] - 1) * (size_t)C;
      for (int j = lane; j < nc; j += 64) {
        float v[8];
        load8<BF16>(x, base + 8 * (size_t)j, v);
        const f32x4_t w0 = *(const f32x4_t*)(w + 8 * j), w1 = *(const f32x4_t*)(w + 8 * j + 4);
        acc += v[0] * w0[0] + v[1] * w0[1] + v[2] * w0[2] + v[3] * w0[3];
        acc += v[4] * w1[0] + v[5] * w1[1] + v[6] * w1[2] + v[7] * w1[3];
      }
      acc = group_sum(acc, 64);
    }
    if (lane == 0) {
      score[s] = option ? acc * inv_sqrt_c : 0.f;
      if (!option) prob[s] = 0.f;
    }
  }
}

// Probabilities: one wave per segment p that has children (grid-stride). The
// children of p lie in (p, S) but need not be contiguous, so the wave scans
// parent[] from p's lowest-index child on, 64 segments per step, each lane
// keeping a running maximum and a sum of exponentials rescaled to it; the 64
// partial (max, sum) pairs are then combined by a butterfly, and a second
// scan writes exp(score - max) / sum for every option of the group. The order
// of every reduction is fixed, so results are deterministic.
__global__ void __launch_bounds__(kMixThreads) readout_softmax_kernel(const int32_t* __restrict__ blob,
                                                                      const float* __restrict__ score,
                                                                      float* __restrict__ prob, BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const int S = blob[MH_S];
  const int32_t* parent = blob + blob[MH_OFF_PARENT];
  const int32_t* first_child = blob + blob[MH_OFF_FIRSTCHILD];
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  for (int p = wave; p < S; p += nwaves) {  // uniform over the wave
    const int fc = first_child[p];
    if (fc < 0) continue;
    float m = -INFINITY, l = 0.f;
    for (int s0 = fc; s0 < S; s0 += 64) {
      const int s = s0 + lane;
      if (s < S && parent[s] == p && first_child[s] < 0) {
        const float z = score[s];
        if (z > m) {
          l = l * expf(m - z) + 1.f;  // m = -inf, l = 0 on a lane's first option: 0 * 0 + 1
          m = z;
        } else {
          l += expf(z - m);
        }
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64), l2 = __shfl_xor(l, o, 64);
      const float mx = fmaxf(m, m2);
      // A lane that saw no option holds (-inf, 0) and contributes nothing;
      // the guards keep -inf - -inf out of expf.
      l = (l > 0.f ? l * expf(m - mx) : 0.f) + (l2 > 0.f ? l2 * expf(m2 - mx) : 0.f);
      m = mx;
    }
    const float inv = 1.f / l;  // l = 0 only when no child of p is an option; then nothing is written
    for (int s0 = fc; s0 < S; s0 += 64) {
      const int s = s0 + lane;
      if (s < S && parent[s] == p && first_child[s] < 0) prob[s] = expf(score[s] - m) * inv;
    }
  }
}

int row_grid(long long rows, int L) {
  const long long rows_per_block = (long long)(kMixThreads / 64) * (64 / L);
  const long long want = (rows + rows_per_block - 1) / rows_per_block;
  const long long cap = (long long)device_cu_count() * 16;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

template <bool BF16>
fork_status launch_gate_t(const fork_meta* m, const void* x, const void* g, long long ldg, const float* w, void* y,
                          int nh, int D, int mode, float eps, hipStream_t stream) {
  const int L = lanes_per_row(D);
  const int grid = row_grid((long long)m->caps.t_cap * nh, L);
  const int32_t* blob = (const int32_t*)m->dev;
  if (mode == 0)
    hipLaunchKernelGGL((gate_kernel<BF16, 0>), dim3(grid), dim3(kMixThreads), 0, stream, blob, x, g, ldg, w, y, nh, D, L, eps,
                       blob_guard(m->caps));
  else if (mode == 1)
    hipLaunchKernelGGL((gate_kernel<BF16, 1>), dim3(grid), dim3(kMixThreads), 0, stream, blob, x, g, ldg, w, y, nh, D, L, eps,
                       blob_guard(m->caps));
  else
    hipLaunchKernelGGL((gate_kernel<BF16, 2>), dim3(grid), dim3(kMixThreads), 0, stream, blob, x, g, ldg, w, y, nh, D, L, eps,
                       blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

}  // namespace

fork_status launch_gate(const fork_meta* m, const void* x, const void* g, long long ldg, const float* w, void* y,
                        int nh, int D, int mode, float eps, fork_dtype dt, hipStream_t stream) {
  if (dt == FORK_BF16) return launch_gate_t<true>(m, x, g, ldg, w, y, nh, D, mode, eps, stream);
  return launch_gate_t<false>(m, x, g, ldg, w, y, nh, D, mode, eps, stream);
}

fork_status launch_quantize_fp8(const void* x, void* q, float* scales, long long rows, int K, fork_dtype dt,
                                hipStream_t stream) {
  const int L = lanes_per_row(K);
  const int grid = row_grid(rows, L);
  if (dt == FORK_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<true>, dim3(grid), dim3(kMixThreads), 0, stream, x, (unsigned char*)q, scales,
                       rows, K, L);
  else
    hipLaunchKernelGGL(quant_rows_kernel<false>, dim3(grid), dim3(kMixThreads), 0, stream, x, (unsigned char*)q,
                       scales, rows, K, L);
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

fork_status launch_gdn_inputs(const fork_meta* m, const void* c, const void* ab, long long ld_ab, const float* a_log,
                              const float* dt_bias, void* q, void* k, void* v, float* a, float* b, int H, int dk,
                              int dv, float eps, fork_dtype dt, hipStream_t stream) {
  const int L = c ? lanes_per_row(dk < dv ? dk : dv) : 1;  // decay / strength only: a lane per row
  const int grid = row_grid((long long)m->caps.t_cap * H, L);
  const int32_t* blob = (const int32_t*)m->dev;
  if (dt == FORK_BF16)
    hipLaunchKernelGGL(gdn_inputs_kernel<true>, dim3(grid), dim3(kMixThreads), 0, stream, blob, c, ab, a_log, dt_bias,
                       q, k, v, a, b, H, dk, dv, ld_ab, L, eps, blob_guard(m->caps));
  else
    hipLaunchKernelGGL(gdn_inputs_kernel<false>, dim3(grid), dim3(kMixThreads), 0, stream, blob, c, ab, a_log, dt_bias,
                       q, k, v, a, b, H, dk, dv, ld_ab, L, eps, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}


fork_status launch_readout(const fork_meta* m, const void* x, const float* w, int C, float* score, float* prob,
                           fork_dtype dt, hipStream_t stream) {
  const int32_t* blob = (const int32_t*)m->dev;
  const int grid = row_grid((long long)m->caps.s_cap, 64);  // a wave per segment
  const float inv_sqrt_c = (float)(1.0 / sqrt((double)C));
  if (dt == FORK_BF16)
    hipLaunchKernelGGL(readout_score_kernel<true>, dim3(grid), dim3(kMixThreads), 0, stream, blob, x, w, C,
                       inv_sqrt_c, score, prob, blob_guard(m->caps));
  else
    hipLaunchKernelGGL(readout_score_kernel<false>, dim3(grid), dim3(kMixThreads), 0, stream, blob, x, w, C,
                       inv_sqrt_c, score, prob, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  hipLaunchKernelGGL(readout_softmax_kernel, dim3(grid), dim3(kMixThreads), 0, stream, blob,
                     (const float*)score, prob, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

}  // namespace fork
