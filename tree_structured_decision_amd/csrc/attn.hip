// Tree-masked flash attention over the flattened decision stream (gfx950).
//
// Semantics (Flide, kongchang.com page, sections "attention masks and
// probability distortion" and "ForkAttention: exact forking in GPU indices"):
// token t of segment s attends to every token of s's ancestor segments and to
// the tokens of s up to t; siblings never see each other, so each branch gets
// exactly the softmax of an isolated forward pass.
//
// Work decomposition. A work item is (query tile, kv head). A query tile holds
// up to 128 rows = tokens x GQA heads of one kv head, taken from one segment or
// from several consecutive short sibling segments (which share all ancestor
// keys). The item walks the ancestor segments' key ranges (fully visible, no
// mask except the ragged end of a range) and then its own range (masked by
// seg_start(row) <= j <= t(row)). Every 64-key K/V tile is staged in LDS once
// and used by all 128 rows, so a long shared prefix is read once per tile of
// packed branch queries instead of once per branch.
//
// Kernel shape: 256 threads = 4 wave64s, each wave owns 32 query rows.
// S^T = K Q^T and O^T = V^T P^T on MFMA (32x32x16 bf16, or 32x32x2 f32): with
// keys on the MFMA M dimension, each lane holds one query row's scores in its
// registers, so the online-softmax row max needs one cross-lane step and the
// row sum none until the end. V is written transposed into LDS so that the
// A operand of O^T = V^T P^T reads contiguous keys.
#include <type_traits>

#include "common.h"

namespace fork {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool BF16, int D>
struct AttnCfg {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int EPC = 16 / ESZ;                 // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per K/V row
  static constexpr int KS = D + EPC;                   // Ks row stride (elements)
  static constexpr int VS = kAttnKeys + (BF16 ? 8 : 4);  // Vt row stride (elements)
  static constexpr int NKF = BF16 ? D / 16 : D / 2;    // MFMA k-steps over D
  static constexpr int NDB = D / 32;                   // 32-row d blocks of O^T
};

struct AttnArgs {
  const int32_t* blob;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int H, Hkv, G;
  float scale_log2;  // softmax scale * log2(e)
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Stage keys [j0, j0 + 64) of kv head g: K row-major into Ks, V transposed into
// Vt. Rows past `jmax` repeat row jmax (in range; their scores are masked).
template <bool BF16, int D, typename E>
__device__ __forceinline__ void stage_kv(E* __restrict__ Ks, E* __restrict__ Vt,
                                         const E* __restrict__ K, const E* __restrict__ V,
                                         int j0, int jmax, int g, int Hkv, int tid) {
  using C = AttnCfg<BF16, D>;
#pragma unroll
  for (int task = tid; task < kAttnKeys * C::CPR; task += 256) {
    const int row = task / C::CPR, ch = task % C::CPR;
    const int j = min(j0 + row, jmax);
    const u32x4_t val = *(const u32x4_t*)(K + ((size_t)j * Hkv + g) * D + ch * C::EPC);
    *(u32x4_t*)(Ks + row * C::KS + ch * C::EPC) = val;
  }
#pragma unroll
  for (int task = tid; task < (kAttnKeys / 4) * C::CPR; task += 256) {
    const int kq = task / C::CPR, ch = task % C::CPR;
    u32x4_t x[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = min(j0 + 4 * kq + jj, jmax);
      x[jj] = *(const u32x4_t*)(V + ((size_t)j * Hkv + g) * D + ch * C::EPC);
    }
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = i >> 1, sh = (i & 1) * 16;
        const unsigned e0 = (x[0][w] >> sh) & 0xffffu, e1 = (x[1][w] >> sh) & 0xffffu;
        const unsigned e2 = (x[2][w] >> sh) & 0xffffu, e3 = (x[3][w] >> sh) & 0xffffu;
        uint2 pk;
        pk.x = e0 | (e1 << 16);
        pk.y = e2 | (e3 << 16);
        *(uint2*)(Vt + (ch * 8 + i) * C::VS + 4 * kq) = pk;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4_t pk;
        pk[0] = x[0][i];
        pk[1] = x[1][i];
        pk[2] = x[2][i];
        pk[3] = x[3][i];
        *(u32x4_t*)(Vt + (ch * 4 + i) * C::VS + 4 * kq) = pk;
      }
    }
  }
}

template <bool BF16, int D>
__global__ void __launch_bounds__(256, 2) fork_attn_kernel(AttnArgs args) {
  using C = AttnCfg<BF16, D>;
  using E = typename std::conditional<BF16, unsigned short, float>::type;
  using QF = typename std::conditional<BF16, bf16x8_t, float>::type;
  __shared__ __attribute__((aligned(16))) E Ks[kAttnKeys * C::KS];
  __shared__ __attribute__((aligned(16))) E Vt[D * C::VS];

  const int32_t* __restrict__ blob = args.blob;
  const int ntiles = blob[MH_NTILES];
  const int TT = blob[MH_TILE_TOKENS];
  const AttnTile* __restrict__ tiles = (const AttnTile*)(blob + blob[MH_OFF_TILES]);
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int32_t* __restrict__ tok_pos = blob + blob[MH_OFF_TOKPOS];
  const E* __restrict__ Q = (const E*)args.q;
  const E* __restrict__ K = (const E*)args.k;
  const E* __restrict__ V = (const E*)args.v;
  E* __restrict__ O = (E*)args.o;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int H = args.H, Hkv = args.Hkv, G = args.G;
  const int nitems = ntiles * Hkv;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int ti = item / Hkv, g = item - ti * Hkv;
    const AttnTile tile = tiles[ti];

    // this lane's query row (rows past the tile are clamped and not stored)
    const int r = wave * 32 + l32;
    const int tl = r / G, hg = r - tl * G;
    const bool valid = tl < TT && tile.t0 + tl < tile.t1;
    const int t_row = valid ? tile.t0 + tl : tile.t1 - 1;
    const int h = g * G + (valid ? hg : 0);
    const int lo_row = t_row - tok_pos[t_row];

    QF qf[C::NKF];
    {
      const E* qrow = Q + ((size_t)t_row * H + h) * D;
#pragma unroll
      for (int ks = 0; ks < C::NKF; ++ks) {
        if constexpr (BF16)
          qf[ks] = *(const bf16x8_t*)(qrow + 16 * ks + 8 * hi);
        else
          qf[ks] = qrow[2 * ks + hi];
      }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

    // one 64-key tile of range [lo, hi_): own == tree-masked own range
    auto kv_tile = [&](int j0, int hi_, bool own) {
      __syncthreads();  // previous tile fully consumed
      stage_kv<BF16, D, E>(Ks, Vt, K, V, j0, hi_ - 1, g, Hkv, tid);
      __syncthreads();

      f32x16_t s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[b][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::NKF; ++ks) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if constexpr (BF16) {
            const bf16x8_t a = *(const bf16x8_t*)(Ks + (32 * b + l32) * C::KS + 16 * ks + 8 * hi);
            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[b], 0, 0, 0);
          } else {
            const float a = Ks[(32 * b + l32) * C::KS + 2 * ks + hi];
            s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[ks], s[b], 0, 0, 0);
          }
        }
      }

      // scale, mask, online softmax (scores in log2 units)
      const bool need_mask = own ? ((tile.info & kTileMulti) != 0 || j0 + kAttnKeys > tile.t0)
                                 : (j0 + kAttnKeys > hi_);
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[b][i] * args.scale_log2;
          if (need_mask) {
            const int j = j0 + 32 * b + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = j < hi_ && (!own || (j >= lo_row && j <= t_row));
            x = vis ? x : -INFINITY;
          }
          s[b][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[b][i] - m_use);
          s[b][i] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if constexpr (BF16) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            bf16x8_t pb;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) pb[jj] = (__bf16)s[b][8 * hf + jj];
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
              const E* vrow = Vt + (32 * db + l32) * C::VS + 32 * b + 16 * hf + 4 * hi;
              const uint2 x0 = *(const uint2*)vrow;
              const uint2 x1 = *(const uint2*)(vrow + 8);
              u32x4_t w;
              w[0] = x0.x;
              w[1] = x0.y;
              w[2] = x1.x;
              w[3] = x1.y;
              const bf16x8_t va = __builtin_bit_cast(bf16x8_t, w);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * b + 8 * (i >> 2) + 4 * hi + (i & 3);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
              const float va = Vt[(32 * db + l32) * C::VS + key];
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[b][i], oacc[db], 0, 0, 0);
            }
          }
        }
      }
    };

    // ancestors: each fully visible
    for (int a = (tile.info & kTileAncMask) - 1; a >= 0; a = parent[a]) {
      const int lo = seg_start[a], hi_ = lo + seg_len[a];
      for (int j0 = lo; j0 < hi_; j0 += kAttnKeys) kv_tile(j0, hi_, false);
    }
    // own range, tree-masked
    for (int j0 = tile.own_lo; j0 < tile.t1; j0 += kAttnKeys) kv_tile(j0, tile.t1, true);

    // finalize
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (valid) {
      E* orow = O + ((size_t)t_row * H + h) * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = 32 * db + 8 * rq + 4 * hi;
          const float v0 = oacc[db][4 * rq + 0] * inv, v1 = oacc[db][4 * rq + 1] * inv;
          const float v2 = oacc[db][4 * rq + 2] * inv, v3 = oacc[db][4 * rq + 3] * inv;
          if constexpr (BF16) {
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            bf16x2_t p0, p1;
            p0[0] = (__bf16)v0;
            p0[1] = (__bf16)v1;
            p1[0] = (__bf16)v2;
            p1[1] = (__bf16)v3;
            uint2 pk;
            pk.x = __builtin_bit_cast(unsigned, p0);
            pk.y = __builtin_bit_cast(unsigned, p1);
            *(uint2*)(orow + d0) = pk;
          } else {
            *(float4*)(orow + d0) = make_float4(v0, v1, v2, v3);
          }
        }
      if (args.lse && hi == 0) args.lse[(size_t)t_row * H + h] = m_run * 0.6931471805599453f + __logf(l_tot);
    }
  }
}

template <bool BF16, int D>
fork_status launch_one(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fork_attn_kernel<BF16, D>), dim3(grid), dim3(256), 0, stream, a);
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

}  // namespace

fork_status launch_attention(const fork_meta* m, const void* q, const void* k, const void* v, void* o,
                             float* lse, int H, int Hkv, int D, float scale, fork_dtype dt,
                             hipStream_t stream) {
  AttnArgs a;
  a.blob = (const int32_t*)m->dev;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  // Persistent grid: two workgroups per CU. Under capture the tree can change
  // between replays, so the grid must not depend on the current tile count.
  int grid = 2 * device_cu_count();
  if (!stream_capturing(stream)) {
    const long long items = (long long)m->num_attn_tiles * Hkv;
    if (items < grid) grid = (int)(items > 0 ? items : 1);
  }
  if (dt == FORK_BF16) return D == 128 ? launch_one<true, 128>(a, grid, stream) : launch_one<true, 64>(a, grid, stream);
  return D == 128 ? launch_one<false, 128>(a, grid, stream) : launch_one<false, 64>(a, grid, stream);
}

}  // namespace fork
