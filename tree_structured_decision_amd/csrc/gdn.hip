// Forked Gated DeltaNet over the flattened decision stream (gfx950).
//
// Per head the dv x dk state follows S_t = a_t S_{t-1} (I - b_t k_t k_t^T) +
// b_t v_t k_t^T with output o_t = scale * S_t q_t. Each segment starts from its
// parent's end state, copied exactly into the segment's start slot (the fork;
// techfi24.com page, "Exact State Forking"; kongchang.com page, "Gated
// DeltaNet layer": every branch's state evolves in the isolated update order).
//
// Chunked form (chunks of 64 tokens that never cross a segment boundary). With
// g_i the in-chunk cumulative sum of log a, gamma_i = exp(g_i), S0 the state
// before the chunk:
//   A   = strictly_lower(diag(b) (K K^T) * exp(g_i - g_j)),  T = (I + A)^-1
//   T'' = T diag(b)
//   U   = T'' (V - diag(gamma) K S0^T)
//   O   = diag(gamma) Q S0^T + (Q K^T * Gamma) U,  Gamma_ij = exp(g_i - g_j), j <= i
//   S_C = gamma_C S0 + U^T diag(gamma_C / gamma) K
// (derived by unrolling the recurrence; u_t = b_t (v_t - a_t S_{t-1} k_t)).
//
// Kernels:
//   gdn_prep: one workgroup per (chunk, head), fully parallel. Computes g,
//     T'' and Q K^T * Gamma into the workspace.
//   gdn_scan: one launch per tree depth. A work item is (segment, head,
//     16-row slice of the state); rows of the state evolve independently, so
//     slices need no communication. It walks its segment's chunks serially
//     and at the end writes its final state into the first child's start
//     slot; the other children copy it from there at the next depth.
//
// Precision. In bf16 mode q/k/v are exact bf16, so products with them as the
// only rounded-free operands use one bf16 MFMA; operands that are computed in
// fp32 (the state, T'', Q K^T * Gamma, U) are split into bf16 hi + lo parts and
// multiplied with hi*hi + hi*lo + lo*hi, which keeps about 16 mantissa bits
// (the usual operand-splitting refinement for low-precision matrix units). The
// state stays fp32 in registers. fp32 mode uses fp32 MFMA throughout.
#include <type_traits>

#include "common.h"

namespace fork {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int CH = kChunk;  // 64
constexpr int VSL = 16;     // state rows per scan work item

// Per (chunk, head) workspace block: T'' [64x64] and P = QK^T*Gamma [64x64],
// each as bf16 hi/lo planes (bf16 mode) or one fp32 plane (fp32 mode), then g.
constexpr size_t kWsPlane = (size_t)CH * CH * 4;  // bytes of one 64x64 operand
constexpr size_t kWsChunk = 2 * kWsPlane + 256;   // T'', P, g (64 floats)

template <bool BF16>
struct GT {
  using E = typename std::conditional<BF16, unsigned short, float>::type;
  using F = typename std::conditional<BF16, bf16x8_t, float>::type;
  static constexpr int KSTEP = BF16 ? 32 : 4;  // k per 16x16 MFMA
  static constexpr int EPC = BF16 ? 8 : 4;     // elements per 16-byte chunk
  static constexpr int PAD = BF16 ? 8 : 4;
};

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
__device__ __forceinline__ float bf16_val(unsigned short u) {
  return __uint_as_float((unsigned)u << 16);
}
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_val(hi));
}

// A/B fragment of an operand stored row-major with k contiguous: lane holds
// (row, k0 + slice) where slice = lane / 16.
template <bool BF16>
__device__ __forceinline__ typename GT<BF16>::F ld_rowk(const typename GT<BF16>::E* base, int ld, int row,
                                                        int k0, int kq) {
  if constexpr (BF16)
    return *(const bf16x8_t*)(base + row * ld + k0 + 8 * kq);
  else
    return base[row * ld + k0 + kq];
}
// Fragment of an operand stored with k along rows (k-major): element (k, col).
template <bool BF16>
__device__ __forceinline__ typename GT<BF16>::F ld_kcol(const typename GT<BF16>::E* base, int ld, int col,
                                                        int k0, int kq) {
  if constexpr (BF16) {
    bf16x8_t f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      f[jj] = __builtin_bit_cast(__bf16, base[(k0 + 8 * kq + jj) * ld + col]);
    return f;
  } else {
    return base[(k0 + kq) * ld + col];
  }
}
template <bool BF16>
__device__ __forceinline__ f32x4_t mma(typename GT<BF16>::F a, typename GT<BF16>::F b, f32x4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Store a computed fp32 value as a "split" operand element.
template <bool BF16>
__device__ __forceinline__ void put_split(typename GT<BF16>::E* hi, typename GT<BF16>::E* lo, int idx,
                                          float x) {
  if constexpr (BF16) {
    unsigned short h, l;
    split_bf16(x, h, l);
    hi[idx] = h;
    lo[idx] = l;
  } else {
    hi[idx] = x;
  }
}

struct GdnArgs {
  const int32_t* blob;
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const float* root_state;
  void* o;
  float* seg_start;
  float* seg_final;
  unsigned char* ws;
  int H;
  float scale;
  int level;
};

// ---------------------------------------------------------------------------
// Prep: per (chunk, head) compute g, T'' = (I + A)^-1 diag(b), P = QK^T * Gamma.
template <bool BF16, int DK>
__global__ void __launch_bounds__(256) gdn_prep_kernel(const int32_t* __restrict__ blob, GdnArgs args) {
  using G = GT<BF16>;
  using E = typename G::E;
  constexpr int LDK = DK + G::PAD;
  constexpr int LDA = CH + 4;  // fp32 64x64 tiles
  __shared__ __attribute__((aligned(16))) E Ks[CH * LDK];
  __shared__ __attribute__((aligned(16))) E Qs[CH * LDK];
  __shared__ float As[CH * LDA];
  __shared__ float Ts[CH * LDA];
  __shared__ float Zs[4][16 * 20];
  __shared__ float gs[CH], bs[CH];

  const int nchunks = blob[MH_NCHUNKS];
  const int2* __restrict__ chunks = (const int2*)(blob + blob[MH_OFF_CHUNKS]);
  const int H = args.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, q4 = lane >> 4;
  const E* __restrict__ Kg = (const E*)args.k;
  const E* __restrict__ Qg = (const E*)args.q;

  // registers of the next item: its k and q rows, a and b (prefetched while
  // the current item computes)
  constexpr int CPR = DK / G::EPC;
  constexpr int KL = CH * CPR / 256;
  u32x4_t rk[KL], rq[KL];
  float ra = 1.f, rb = 0.f;
  int rlen = 0;
  // rows past the chunk are clamped to its last row (in range) and zeroed at
  // the LDS store, so no load sits in a divergent branch
  auto prep_load = [&](int item) {
    const int c = item / H, h = item - c * H;
    const int2 ck = chunks[c];
    rlen = ck.y;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int task = tid + 256 * i, row = min(task / CPR, ck.y - 1), ch = task % CPR;
      const size_t off = ((size_t)(ck.x + row) * H + h) * DK + ch * G::EPC;
      rk[i] = *(const u32x4_t*)(Kg + off);
      rq[i] = *(const u32x4_t*)(Qg + off);
    }
    const size_t ab = (size_t)(ck.x + min(tid & (CH - 1), ck.y - 1)) * H + h;
    ra = args.a[ab];
    rb = args.b[ab];
  };
  if (blockIdx.x < nchunks * H) prep_load(blockIdx.x);

  for (int item = blockIdx.x; item < nchunks * H; item += gridDim.x) {
    const int c = item / H, h = item - c * H;
    unsigned char* wsb = args.ws + ((size_t)c * H + h) * kWsChunk;

    __syncthreads();  // LDS reuse across items
    const int len = rlen;
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int task = tid + 256 * i, row = task / CPR, ch = task % CPR;
      *(u32x4_t*)(Ks + row * LDK + ch * G::EPC) = row < len ? rk[i] : z4;
      *(u32x4_t*)(Qs + row * LDK + ch * G::EPC) = row < len ? rq[i] : z4;
    }
    if (w == 0) {
      // g = inclusive cumulative sum of log a (padding: a = 1, b = 0)
      const int i = lane;
      float la = i < len ? logf(ra) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off);
        if (i >= off) la += y;
      }
      gs[i] = la;
      bs[i] = i < len ? rb : 0.f;
      ((float*)(wsb + 2 * kWsPlane))[i] = la;
    }
    // zero Ts (upper blocks stay zero)
    for (int i = tid; i < CH * LDA; i += 256) Ts[i] = 0.f;
    __syncthreads();
    if (item + (int)gridDim.x < nchunks * H) prep_load(item + gridDim.x);

    // K K^T -> A (strictly lower, scaled);  Q K^T -> P (lower incl. diagonal)
    {
      E* Ph = (E*)(wsb + kWsPlane);
      E* Pl = BF16 ? (E*)(wsb + kWsPlane) + CH * CH : nullptr;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        f32x4_t kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += G::KSTEP) {
          const typename G::F bK = ld_rowk<BF16>(Ks, LDK, 16 * J + c16, k0, q4);
          kk = mma<BF16>(ld_rowk<BF16>(Ks, LDK, 16 * w + c16, k0, q4), bK, kk);
          qk = mma<BF16>(ld_rowk<BF16>(Qs, LDK, 16 * w + c16, k0, q4), bK, qk);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * w + 4 * q4 + r, j = 16 * J + c16;
          const float dec = j <= i ? __expf(gs[i] - gs[j]) : 0.f;
          As[i * LDA + j] = j < i ? bs[i] * dec * kk[r] : 0.f;
          put_split<BF16>(Ph, Pl, i * CH + j, dec * qk[r]);
        }
      }
    }
    __syncthreads();

    // diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution
    if (lane < 16) {
      const int base = 16 * w, col = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= As[(base + i) * LDA + base + j] * x[j];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(base + i) * LDA + base + col] = x[i];
    }
    __syncthreads();

    // off-diagonal blocks: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ, by distance
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      const int I = w + dist, J = w;
      const bool act = I < 4;
      f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      if (act) {
        for (int Kb = J; Kb < I; ++Kb)
#pragma unroll
          for (int k0 = 0; k0 < 16; k0 += 4)
            z = mma_f32(As[(16 * I + c16) * LDA + 16 * Kb + k0 + q4],
                        Ts[(16 * Kb + k0 + q4) * LDA + 16 * J + c16], z);
#pragma unroll
        for (int r = 0; r < 4; ++r) Zs[w][(4 * q4 + r) * 20 + c16] = z[r];
      }
      __syncthreads();
      if (act) {
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
          t = mma_f32(Ts[(16 * I + c16) * LDA + 16 * I + k0 + q4], Zs[w][(k0 + q4) * 20 + c16], t);
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[(16 * I + 4 * q4 + r) * LDA + 16 * J + c16] = -t[r];
      }
      __syncthreads();
    }

    // T'' = T diag(b) -> workspace
    {
      E* Th = (E*)wsb;
      E* Tl = BF16 ? (E*)wsb + CH * CH : nullptr;
      for (int idx = tid; idx < CH * CH; idx += 256) {
        const int i = idx >> 6, j = idx & 63;
        put_split<BF16>(Th, Tl, idx, Ts[i * LDA + j] * bs[j]);
      }
    }
  }
}

// Everything one scan chunk reads from global memory, in registers between
// its loads (issued while the previous chunk computes) and its use. K is the
// only chunk operand every wave needs in full, so it alone goes through LDS;
// the other operands are loaded directly in the MFMA fragment layout of the
// wave that uses them: rows 16w..16w+15 of Q, T'' and P as A fragments, and
// v and g at the rows of this lane's accumulator elements.
template <bool BF16, int DK>
struct ChunkRegs {
  using G = GT<BF16>;
  using F = typename G::F;
  static constexpr int KL = CH * (DK / G::EPC) / 256;  // 16-byte K loads per thread
  static constexpr int NQ = DK / G::KSTEP;             // Q fragments (k-steps over dk)
  static constexpr int NT = CH / G::KSTEP;             // T'', P fragments (k-steps over the chunk)
  static constexpr int NP = BF16 ? 2 : 1;              // hi/lo planes
  u32x4_t k[KL];
  F q[NQ];
  F t[NP][NT], p[NP][NT];
  // one 32-bit register per v element: packing two 16-bit loads into one
  // register would wait for them (and, the counter being in order, for every
  // load issued before them)
  typename std::conditional<BF16, unsigned, float>::type v[4];
  float g[4], gl;
};

// Issues every load of chunk (t0, len) for head h and state slice e0. Rows past
// len are clamped to the chunk's last row: they only meet zero coefficients
// (b = 0 there, so T'' has zero columns and U zero rows) or produce output rows
// that are never stored, so they need no masking and no load is divergent.
template <bool BF16, int DK>
__device__ __forceinline__ void chunk_load(ChunkRegs<BF16, DK>& r, const typename GT<BF16>::E* __restrict__ Kg,
                                           const typename GT<BF16>::E* __restrict__ Qg,
                                           const typename GT<BF16>::E* __restrict__ Vg,
                                           const unsigned char* __restrict__ wsb, int t0, int len, int H, int h,
                                           int e0, int tid) {
  using G = GT<BF16>;
  using R = ChunkRegs<BF16, DK>;
  using E = typename G::E;
  constexpr int CPR = DK / G::EPC;
  const int lane = tid & 63, w = tid >> 6, c16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < R::KL; ++i) {
    const int task = tid + 256 * i, row = min(task / CPR, len - 1), ch = task % CPR;
    r.k[i] = *(const u32x4_t*)(Kg + ((size_t)(t0 + row) * H + h) * DK + ch * G::EPC);
  }
  const int arow = 16 * w + c16;  // A-fragment row of this lane
  {
    const E* qrow = Qg + ((size_t)(t0 + min(arow, len - 1)) * H + h) * DK;
#pragma unroll
    for (int f = 0; f < R::NQ; ++f) {
      if constexpr (BF16)
        r.q[f] = *(const bf16x8_t*)(qrow + f * G::KSTEP + 8 * q4);
      else
        r.q[f] = qrow[f * G::KSTEP + q4];
    }
  }
  const int kend = 16 * (w + 1);  // T'' and P are lower triangular
#pragma unroll
  for (int pl = 0; pl < R::NP; ++pl) {
    const E* Tw = (const E*)wsb + pl * CH * CH + arow * CH;
    const E* Pw = (const E*)(wsb + kWsPlane) + pl * CH * CH + arow * CH;
#pragma unroll
    for (int f = 0; f < R::NT; ++f) {
      if (f * G::KSTEP < kend) {
        if constexpr (BF16) {
          r.t[pl][f] = *(const bf16x8_t*)(Tw + f * G::KSTEP + 8 * q4);
          r.p[pl][f] = *(const bf16x8_t*)(Pw + f * G::KSTEP + 8 * q4);
        } else {
          r.t[pl][f] = Tw[f * G::KSTEP + q4];
          r.p[pl][f] = Pw[f * G::KSTEP + q4];
        }
      }
    }
  }
  const float* gw = (const float*)(wsb + 2 * kWsPlane);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 16 * w + 4 * q4 + j;  // accumulator row of element j
    r.v[j] = Vg[((size_t)(t0 + min(i, len - 1)) * H + h) * DK + e0 + c16];
    r.g[j] = gw[i];
  }
  r.gl = gw[CH - 1];
}

// ---------------------------------------------------------------------------
// Scan: one launch per depth; items (segment, head, 16-row state slice).
template <bool BF16, int DK>
__global__ void __launch_bounds__(256) gdn_scan_kernel(const int32_t* __restrict__ blob, GdnArgs args) {
  using G = GT<BF16>;
  using E = typename G::E;
  using F = typename G::F;
  using R = ChunkRegs<BF16, DK>;
  constexpr int DV = DK;
  constexpr int NS = DV / VSL;       // slices per head
  constexpr int LDK = DK + G::PAD;   // K tile
  constexpr int LDSS = DK + G::PAD;  // state slice
  constexpr int LDR = CH + G::PAD;   // transposed R, U, U'
  constexpr int NDB = DK / 16;       // 16-col d blocks of the state slice
  constexpr int DBW = (NDB + 3) / 4; // d blocks per wave
  constexpr bool SPLIT = BF16;
  constexpr int CPR = DK / G::EPC;
  __shared__ __attribute__((aligned(16))) E Ks[CH * LDK];
  __shared__ __attribute__((aligned(16))) E Sh[VSL * LDSS];
  __shared__ __attribute__((aligned(16))) E Sl[SPLIT ? VSL * LDSS : 8];
  __shared__ __attribute__((aligned(16))) E Rh[VSL * LDR];
  __shared__ __attribute__((aligned(16))) E Rl[SPLIT ? VSL * LDR : 8];
  __shared__ __attribute__((aligned(16))) E Uh[VSL * LDR];
  __shared__ __attribute__((aligned(16))) E Ul[SPLIT ? VSL * LDR : 8];
  __shared__ __attribute__((aligned(16))) E U2h[VSL * LDR];
  __shared__ __attribute__((aligned(16))) E U2l[SPLIT ? VSL * LDR : 8];

  const int level = args.level;
  if (level > blob[MH_MAXDEPTH]) return;
  const int32_t* __restrict__ level_off = blob + blob[MH_OFF_LEVELOFF];
  const int32_t* __restrict__ level_seg = blob + blob[MH_OFF_LEVELSEG];
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ root_ord = blob + blob[MH_OFF_ROOTORD];
  const int32_t* __restrict__ first_child = blob + blob[MH_OFF_FIRSTCHILD];
  const int32_t* __restrict__ chunk_base = blob + blob[MH_OFF_CHUNKBASE];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int lv0 = level_off[level], nlev = level_off[level + 1] - lv0;
  const int H = args.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, q4 = lane >> 4;
  const E* __restrict__ Kg = (const E*)args.k;
  const E* __restrict__ Qg = (const E*)args.q;
  const E* __restrict__ Vg = (const E*)args.v;
  E* __restrict__ Og = (E*)args.o;
  const size_t SZ = (size_t)DV * DK;
  const int kend = 16 * (w + 1);  // T'' and P are lower triangular

  // Work items: (segment, head, slice). Workgroups are dispatched round-robin
  // over the 8 XCDs (workgroup id mod 8; the grid is a multiple of 8), so item
  // i runs on XCD i mod 8. Heads are assigned so that all slices of one head
  // run on the same XCD and share its L2 for the chunk operands (k, q, T'', P)
  // they all read.
  const int NH8 = (H + 7) / 8;
  for (int item = blockIdx.x; item < nlev * NH8 * 8 * NS; item += gridDim.x) {
    const int x = item & 7, j = item >> 3;
    const int sl = j % NS, j2 = j / NS;
    const int h = (j2 % NH8) * 8 + x, li = j2 / NH8;
    if (h >= H) continue;
    // per-item metadata, uniform across the workgroup (scalar loads)
    const int s = __builtin_amdgcn_readfirstlane(level_seg[lv0 + li]);
    const int e0 = sl * VSL;
    const int p = __builtin_amdgcn_readfirstlane(parent[s]);
    const int L = __builtin_amdgcn_readfirstlane(seg_len[s]);
    const int st = __builtin_amdgcn_readfirstlane(seg_start[s]);
    const int cb = __builtin_amdgcn_readfirstlane(chunk_base[s]);
    const int fc_p = p >= 0 ? __builtin_amdgcn_readfirstlane(first_child[p]) : -1;
    const int ro = p < 0 ? __builtin_amdgcn_readfirstlane(root_ord[s]) : 0;
    // chunk ci of the segment covers tokens [st + 64 ci, st + min(64 (ci + 1), L))
    const int nck = (L + CH - 1) / CH;

    // ---- start state: root_state / zero, or the parent's end state (read from
    // the first child's start slot, where the parent's scan left it)
    const float* src = nullptr;
    float* dst = nullptr;
    float* own_slot = args.seg_start + ((size_t)s * H + h) * SZ;
    if (p < 0) {
      if (args.root_state) src = args.root_state + ((size_t)ro * H + h) * SZ;
      dst = own_slot;
    } else {
      src = args.seg_start + ((size_t)fc_p * H + h) * SZ;
      if (fc_p != s) dst = own_slot;
    }
    // branch-free loads from an always-valid address; zero when there is no source
    const bool has_src = src != nullptr;
    const float* lsrc = has_src ? src : own_slot;
    f32x4_t Sreg[DBW];
#pragma unroll
    for (int bi = 0; bi < DBW; ++bi) {
      const int db = min(w * DBW + bi, NDB - 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = lsrc[(size_t)(e0 + 4 * q4 + r) * DK + 16 * db + c16];
        Sreg[bi][r] = has_src ? x : 0.f;
      }
    }
    // first chunk's loads go out together with the state loads
    R nx;
    chunk_load<BF16, DK>(nx, Kg, Qg, Vg, args.ws + ((size_t)cb * H + h) * kWsChunk, st, min(CH, L), H, h, e0,
                         tid);
    if (dst) {
#pragma unroll
      for (int bi = 0; bi < DBW; ++bi) {
        const int db = w * DBW + bi;
        if (db < NDB)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(size_t)(e0 + 4 * q4 + r) * DK + 16 * db + c16] = Sreg[bi][r];
      }
    }

    // output rows of the previous chunk, stored one iteration late (after the
    // next chunk's loads are issued)
    float oval[4] = {0.f, 0.f, 0.f, 0.f};
    int orow0 = 0, olen = 0;
    auto flush_o = [&]() {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * q4 + r;
        if (i < olen) {
          E* d = Og + ((size_t)(orow0 + i) * H + h) * DV + e0 + c16;
          if constexpr (BF16) *d = bf16_bits(oval[r]); else *d = oval[r];
        }
      }
    };

    for (int ci = 0; ci < nck; ++ci) {
      const int c = cb + ci;
      const int t0 = st + CH * ci, len = min(CH, L - CH * ci);
      R cur = nx;  // this chunk's operands

      __syncthreads();  // previous chunk done with Ks, Sh/Sl and the exchange tiles
#pragma unroll
      for (int i = 0; i < R::KL; ++i) {
        const int task = tid + 256 * i, row = task / CPR, ch = task % CPR;
        *(u32x4_t*)(Ks + row * LDK + ch * G::EPC) = cur.k[i];
      }
#pragma unroll
      for (int bi = 0; bi < DBW; ++bi) {
        const int db = w * DBW + bi;
        if (db < NDB)
#pragma unroll
          for (int r = 0; r < 4; ++r) put_split<BF16>(Sh, Sl, (4 * q4 + r) * LDSS + 16 * db + c16, Sreg[bi][r]);
      }
      float gam[4], rr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gam[r] = __expf(cur.g[r]);
        rr[r] = __expf(cur.gl - cur.g[r]);
      }
      const float gC = __expf(cur.gl);
      __syncthreads();
      // next chunk's loads first, then the previous chunk's output stores: a
      // load issued after a possibly aliasing store waits for that store, so
      // stores go out a whole chunk ahead of the next loads
      if (ci + 1 < nck)
        chunk_load<BF16, DK>(nx, Kg, Qg, Vg, args.ws + ((size_t)(c + 1) * H + h) * kWsChunk, t0 + CH,
                             min(CH, L - CH * (ci + 1)), H, h, e0, tid);
      flush_o();

      // (1) X = K S^T, Y = Q S^T   (rows 16w.., cols e); separate hi/lo chains
      f32x4_t X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
      f32x4_t X2 = {0.f, 0.f, 0.f, 0.f}, Y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < R::NQ; ++f) {
        const int k0 = f * G::KSTEP;
        const F aK = ld_rowk<BF16>(Ks, LDK, 16 * w + c16, k0, q4);
        const F bh = ld_rowk<BF16>(Sh, LDSS, c16, k0, q4);
        X = mma<BF16>(aK, bh, X);
        Y = mma<BF16>(cur.q[f], bh, Y);
        if constexpr (SPLIT) {
          const F bl = ld_rowk<BF16>(Sl, LDSS, c16, k0, q4);
          X2 = mma<BF16>(aK, bl, X2);
          Y2 = mma<BF16>(cur.q[f], bl, Y2);
        }
      }
      // (2) R = V - gamma * X  -> R^T
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * q4 + r;
        float vv;
        if constexpr (BF16) vv = __uint_as_float(cur.v[r] << 16); else vv = cur.v[r];
        put_split<BF16>(Rh, Rl, c16 * LDR + i, vv - gam[r] * (X[r] + X2[r]));
      }
      __syncthreads();

      // (3) U = T'' R  (T'' lower triangular: k < 16(w+1))
      f32x4_t Ua = {0.f, 0.f, 0.f, 0.f}, Ub = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < R::NT; ++f) {
        const int k0 = f * G::KSTEP;
        if (k0 < kend) {
          const F bh = ld_rowk<BF16>(Rh, LDR, c16, k0, q4);
          Ua = mma<BF16>(cur.t[0][f], bh, Ua);
          if constexpr (SPLIT) {
            Ub = mma<BF16>(cur.t[0][f], ld_rowk<BF16>(Rl, LDR, c16, k0, q4), Ub);
            Ub = mma<BF16>(cur.t[SPLIT ? 1 : 0][f], bh, Ub);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * q4 + r;
        const float u = Ua[r] + Ub[r];
        put_split<BF16>(Uh, Ul, c16 * LDR + i, u);
        put_split<BF16>(U2h, U2l, c16 * LDR + i, u * rr[r]);
      }
      __syncthreads();

      // (4) O = scale * (gamma * Y + P U), stored at the next iteration
      {
        f32x4_t Za = {0.f, 0.f, 0.f, 0.f}, Zb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < R::NT; ++f) {
          const int k0 = f * G::KSTEP;
          if (k0 < kend) {
            const F bh = ld_rowk<BF16>(Uh, LDR, c16, k0, q4);
            Za = mma<BF16>(cur.p[0][f], bh, Za);
            if constexpr (SPLIT) {
              Zb = mma<BF16>(cur.p[0][f], ld_rowk<BF16>(Ul, LDR, c16, k0, q4), Zb);
              Zb = mma<BF16>(cur.p[SPLIT ? 1 : 0][f], bh, Zb);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) oval[r] = args.scale * (gam[r] * (Y[r] + Y2[r]) + Za[r] + Zb[r]);
        orow0 = t0;
        olen = len;
      }
      // (5) S = gamma_C S + U'^T K
#pragma unroll
      for (int bi = 0; bi < DBW; ++bi) {
        const int db = w * DBW + bi;
        if (db < NDB) {
          f32x4_t acc = Sreg[bi] * gC;
          f32x4_t acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0 = 0; k0 < CH; k0 += G::KSTEP) {
            const F bk = ld_kcol<BF16>(Ks, LDK, 16 * db + c16, k0, q4);
            acc = mma<BF16>(ld_rowk<BF16>(U2h, LDR, c16, k0, q4), bk, acc);
            if constexpr (SPLIT) acc2 = mma<BF16>(ld_rowk<BF16>(U2l, LDR, c16, k0, q4), bk, acc2);
          }
          Sreg[bi] = acc + acc2;
        }
      }
    }
    flush_o();

    // ---- end state: seg_final_state and the first child's start slot (the fork)
    {
      const int fc = __builtin_amdgcn_readfirstlane(first_child[s]);
      float* d1 = args.seg_final ? args.seg_final + ((size_t)s * H + h) * SZ : nullptr;
      float* d2 = fc >= 0 ? args.seg_start + ((size_t)fc * H + h) * SZ : nullptr;
#pragma unroll
      for (int bi = 0; bi < DBW; ++bi) {
        const int db = w * DBW + bi;
        if (db < NDB)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const size_t idx = (size_t)(e0 + 4 * q4 + r) * DK + 16 * db + c16;
            if (d1) d1[idx] = Sreg[bi][r];
            if (d2) d2[idx] = Sreg[bi][r];
          }
      }
    }
  }
}

template <bool BF16, int DK>
fork_status launch_gdn_t(const fork_meta* m, GdnArgs a, hipStream_t stream) {
  const bool cap = stream_capturing(stream);
  const int cus = device_cu_count();
  int grid = 2 * cus;
  if (!cap) {
    const long long items = (long long)m->num_chunks * a.H;
    if (items < grid) grid = (int)(items > 0 ? items : 1);
  }
  hipLaunchKernelGGL((gdn_prep_kernel<BF16, DK>), dim3(grid), dim3(256), 0, stream, a.blob, a);
  FORK_HIP_CHECK(hipGetLastError());
  // One scan launch per depth (children start after their parents ended).
  // Under capture, every depth up to the capacity is recorded; depths beyond
  // the current tree exit at once.
  const int levels = cap ? m->caps.depth_cap + 1 : m->max_depth + 1;
  const int sgrid = (2 * cus + 7) / 8 * 8;  // a multiple of 8: item i runs on XCD i mod 8
  for (int lv = 0; lv < levels; ++lv) {
    a.level = lv;
    hipLaunchKernelGGL((gdn_scan_kernel<BF16, DK>), dim3(sgrid), dim3(256), 0, stream, a.blob, a);
    FORK_HIP_CHECK(hipGetLastError());
  }
  return FORK_OK;
}

}  // namespace

size_t gdn_workspace_bytes(const fork_meta* m, int H, int dk, int dv) {
  (void)dk;
  (void)dv;
  const BlobLayout L = blob_layout(m->caps);
  return (size_t)L.chunk_cap * H * kWsChunk;
}

fork_status launch_gdn(const fork_meta* m, const void* q, const void* k, const void* v, const float* a,
                       const float* b, const float* root_state, void* o, float* seg_start_state,
                       float* seg_final_state, int H, int dk, int dv, float scale, fork_dtype dt,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)dv;
  (void)ws_bytes;
  GdnArgs g;
  g.blob = (const int32_t*)m->dev;
  g.q = q;
  g.k = k;
  g.v = v;
  g.a = a;
  g.b = b;
  g.root_state = root_state;
  g.o = o;
  g.seg_start = seg_start_state;
  g.seg_final = seg_final_state;
  g.ws = (unsigned char*)ws;
  g.H = H;
  g.scale = scale;
  g.level = 0;
  if (dt == FORK_BF16) {
    if (dk == 128) return launch_gdn_t<true, 128>(m, g, stream);
    if (dk == 64) return launch_gdn_t<true, 64>(m, g, stream);
    return launch_gdn_t<true, 32>(m, g, stream);
  }
  if (dk == 128) return launch_gdn_t<false, 128>(m, g, stream);
  if (dk == 64) return launch_gdn_t<false, 64>(m, g, stream);
  return launch_gdn_t<false, 32>(m, g, stream);
}

}  // namespace fork
