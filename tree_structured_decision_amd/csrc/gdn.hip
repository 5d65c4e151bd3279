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
//   gdn_coop (bf16) / gdn_scan (fp32): one launch per tree depth. A work
//     item is (segment, head, slice of state rows); rows of the state evolve
//     independently, so slices need no communication. It walks its segment's
//     chunks serially and at the end writes its final state into the first
//     child's start slot; the other children copy it from there at the next
//     depth. gdn_coop splits each chunk of a 16-row slice over several waves
//     (short serial chain per chunk); gdn_scan runs one wave per slice.
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

// Per (chunk, head) workspace block.
// fp32 mode: T'' [64x64] and P = QK^T*Gamma [64x64] as row-major fp32 planes,
// then g (64 floats).
// bf16 mode: T'' and P as MFMA operand fragments, then gamma and gamma_C /
// gamma (64 floats each). A fragment is 1 KB: lane l of a 16x16x32 product
// holds 8 bf16 of row 16 I + l % 16 at columns 32 kf + 4 q + {0..3} and
// 32 kf + 16 + 4 q + {0..3}, q = l / 16 (the reduction order of the scan).
// Both matrices are lower triangular, so row block I keeps only its first
// I / 2 + 1 column steps: 6 fragments, each as a hi and a lo plane
// (fragment (I, kf) at index ((tri(I) + kf) * 2 + plane)).
constexpr size_t kWsPlane = (size_t)CH * CH * 4;  // bytes of one 64x64 fp32 operand
constexpr size_t kWsChunk = 2 * kWsPlane + 256;   // the larger of the two layouts
constexpr int kNtri = 6;                          // fragments of a lower-triangular 64x64 operand
__host__ __device__ constexpr int frag_nk(int I) { return I / 2 + 1; }
__host__ __device__ constexpr int frag_tri(int I) { return I < 3 ? I : 4; }
constexpr size_t kWsFrag = (size_t)kNtri * 2 * 1024;  // bytes of T'' (or P) fragments
constexpr size_t kWsGam = 2 * kWsFrag;                // gamma, then gamma_C / gamma
static_assert(kWsGam + 1024 <= kWsChunk, "bf16 workspace layout fits the block (gates staged as 1 KB)");

// bf16 scans split each depth between two kernels: the depth's long segments
// (more than one chunk; they lead its list) go to the chunk-cooperative kernel
// when all of its work items fit in one round of the grid (a latency-bound
// depth such as a single long prefix); everything else goes to the
// one-wave-per-slice kernel, which has the higher throughput.
__device__ __forceinline__ int coop_take(const int32_t* __restrict__ blob, int level, int H, int dv, int sgrid) {
  const int nlong = blob[blob[MH_OFF_LEVELLONG] + level];
  const long long items = (long long)nlong * ((H + 7) / 8) * 8 * (dv / 16);
  return items <= (long long)sgrid ? nlong : 0;
}
__device__ __forceinline__ int coop_segments(const int32_t* __restrict__ blob, int level, int H, int dv) {
  return coop_take(blob, level, H, dv, (int)gridDim.x);
}

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
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;  // operand of the LDS transpose read

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

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// hi and lo bf16 parts of four floats (one accumulator block of a lane)
__device__ __forceinline__ void split4(const f32x4_t& x, u32x2_t& hi, u32x2_t& lo) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const unsigned w = pack_bf16x2(x[2 * p], x[2 * p + 1]);
    hi[p] = w;
    lo[p] = pack_bf16x2(x[2 * p] - __uint_as_float(w << 16), x[2 * p + 1] - __uint_as_float(w & 0xffff0000u));
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
  int32_t* ctr;  // the blob's scan work counters: next item, finished workgroups
  BlobGuard guard;
  int H;
  float scale;
  int level;
  // the depth's segment range [lv_first, lv_first + lv_count) of the blob's
  // level list and its first lv_take segments for gdn_coop_kernel, when the
  // host planned the launch; lv_first < 0: read everything from the blob
  int lv_first, lv_count, lv_take;
  // gdn_prep_kernel: 1 = only the chunks of the segments gdn_coop_kernel takes
  // (the fused kernel prepares the others itself); sgrid: the scans' grid
  int prep_coop_only, sgrid;
  // FP8 inputs (gdn_fused_kernel<.., true>): q, k, v are E4M3 codes with these
  // per-(token, head) scales [T, H]; no_coop: every segment of a depth goes to
  // the fused kernel
  const float* qs;
  const float* ks;
  const float* vs;
  int no_coop;
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// but not for its global loads still in flight (prefetches of the next work
// item, or loads into LDS of the next task, which are awaited explicitly).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Prep: per (chunk, head) compute g, T'' = (I + A)^-1 diag(b), P = QK^T * Gamma.
//
// The products are formed transposed: wave w computes, for each 16-column
// block J <= w, Pt_J = K_J Q_w^T and At_J = K_J K_w^T. Their accumulators give
// lane (c16, q4) row i = 16 w + c16 of QK^T (or of KK^T) at columns
// j = 16 J + 4 q4 + r, r = 0..3: the elements of a P fragment of row block w in
// the scan's reduction order, so P goes to the workspace straight from
// registers, and a row of A goes to LDS as one 16-byte store per block.
// Blocks J > w lie above the diagonal and are zero.
// T = (I + A)^-1 is then formed block-wise: the four diagonal 16x16 blocks by
// forward substitution (one block per wave), the blocks below the diagonal by
// distance, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ.

// DPP lane moves: row_shr:n, and quad permutations (lane ^ 1, lane ^ 2).
// Lanes without a source read zero.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppRowShr = 0x110;    // + n: row_shr:n (within rows of 16 lanes)
constexpr int kDppQuadXor1 = 0xb1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;   // quad_perm [2,3,0,1]
__device__ __forceinline__ float lane_val(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// log a of a decay gate, floored at -20. A gate a = 0 (the state is
// forgotten at that token) would give -inf, and the chunked form's decay
// ratios exp(g_i - g_j) of prefix sums g would become -inf - (-inf) = NaN.
// With the floor, every decay across such a token is at most e^-20 (about
// 2e-9, far below an fp32 ulp of what it multiplies), and the prefix sums
// stay small enough that ratios between tokens on one side of it keep fp32
// accuracy (a floor of -128, which would give exact zeros, costs ~3e-4 on
// fp32 outputs through the rounding of the larger sums). Gates below e^-20
// act as e^-20: no decay factor moves by more than 2.1e-9.
__device__ __forceinline__ float log_gate(float a) { return fmaxf(logf(a), -20.f); }

// Inclusive prefix sum over the 64 lanes of a wave (within rows of 16 lanes by
// DPP shifts, then each row adds the totals of the rows before it).
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
  x += dpp_mov<kDppRowShr + 1>(x);
  x += dpp_mov<kDppRowShr + 2>(x);
  x += dpp_mov<kDppRowShr + 4>(x);
  x += dpp_mov<kDppRowShr + 8>(x);
  const float r0 = lane_val(x, 15), r1 = lane_val(x, 31), r2 = lane_val(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}

// Diagonal block [b0, b0 + 16)^2 of T = (I + A)^-1 by forward substitution,
// x_i = e_i - sum_{j<i} A_ij x_j for the 16 columns, by one wave with four lanes
// per column (lane = 4 c + p): lane (c, p) owns the unknowns x_{4p+t} of column
// c and holds A[i][b0 + 4p + t] for every row i. Rows are solved in groups of
// four: the sum over the groups already solved is four partial sums added
// across the quad, then the lanes p of the group finish its rows in order.
// A's entries on and above the diagonal are zero.
__device__ __forceinline__ void diag_inverse(const float* __restrict__ As, float* __restrict__ Ts, int lda,
                                             int b0, int lane) {
  const int c = lane >> 2, p = lane & 3;
  f32x4_t a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = *(const f32x4_t*)(As + (b0 + i) * lda + b0 + 4 * p);
  f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    float sm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4_t& ai = a[4 * blk + r];
      float v = ai[0] * x[0] + ai[1] * x[1] + ai[2] * x[2] + ai[3] * x[3];
      v += dpp_mov<kDppQuadXor1>(v);
      v += dpp_mov<kDppQuadXor2>(v);
      sm[r] = v;
    }
    const bool mine = p == blk;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * blk + r;
      float v = (i == c ? 1.f : 0.f) - sm[r];
#pragma unroll
      for (int t = 0; t < r; ++t) v -= a[i][t] * x[t];
      x[r] = mine ? v : x[r];
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) Ts[(b0 + 4 * p + t) * lda + b0 + c] = x[t];
}

template <bool BF16, int DK>
struct PrepCfg {
  using G = GT<BF16>;
  static constexpr int LDK = DK + G::PAD;
  static constexpr int LDA = CH + 4;  // fp32 64x64 tiles
  // K and Q tiles; once the products are formed, the same bytes hold A (fp32)
  static constexpr int KQ_BYTES = 2 * CH * LDK * (int)sizeof(typename G::E);
  static constexpr int KQA_BYTES = KQ_BYTES > CH * LDA * 4 ? KQ_BYTES : CH * LDA * 4;
  static constexpr int LDS = KQA_BYTES + CH * LDA * 4 + 4 * CH * 4;
  // workgroups per CU: as many as the LDS holds, up to 3 (bf16; the register
  // budget of 3 waves per SIMD) or 2 (fp32)
  static constexpr int FIT = 160 * 1024 / LDS;
  static constexpr int WANT = BF16 ? 3 : 2;
  static constexpr int PER_CU = FIT < 1 ? 1 : (FIT < WANT ? FIT : WANT);
};

template <bool BF16, int DK>
__global__ void __launch_bounds__(256, (PrepCfg<BF16, DK>::PER_CU))
    gdn_prep_kernel(const int32_t* __restrict__ blob, GdnArgs args) {
  using G = GT<BF16>;
  using E = typename G::E;
  using C = PrepCfg<BF16, DK>;
  constexpr int LDK = C::LDK, LDA = C::LDA;
  constexpr int NKS = DK / G::KSTEP;  // reduction steps of the products
  __shared__ __attribute__((aligned(16))) unsigned char kqa[C::KQA_BYTES];
  E* Ks = (E*)kqa;
  E* Qs = Ks + CH * LDK;
  float* As = (float*)kqa;
  __shared__ __attribute__((aligned(16))) float Ts[CH * LDA];
  // g and b of the chunk, two copies by item parity (an item's writes never
  // meet the previous item's reads, so items need no barrier between them)
  __shared__ __attribute__((aligned(16))) float gsb[2][CH];
  __shared__ __attribute__((aligned(16))) float bsb[2][CH];

  if (!blob_ok(blob, args.guard)) return;
  const int2* __restrict__ chunks = (const int2*)(blob + blob[MH_OFF_CHUNKS]);
  const int H = args.H;
  // the chunks to prepare: all, or those of the segments gdn_coop_kernel takes
  // (at each depth, its first `take` segments; a handful at most)
  int nchunks = blob[MH_NCHUNKS];
  const int32_t* __restrict__ level_off = blob + blob[MH_OFF_LEVELOFF];
  const int32_t* __restrict__ level_seg = blob + blob[MH_OFF_LEVELSEG];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ chunk_base = blob + blob[MH_OFF_CHUNKBASE];
  const int maxd = blob[MH_MAXDEPTH];
  if (args.prep_coop_only) {
    nchunks = 0;
    for (int lv = 0; lv <= maxd; ++lv) {
      const int take = coop_take(blob, lv, H, DK, args.sgrid);
      for (int k = 0; k < take; ++k) nchunks += (seg_len[level_seg[level_off[lv] + k]] + CH - 1) / CH;
    }
  }
  // chunk index of the n-th prepared chunk
  auto chunk_of = [&](int n) -> int {
    if (!args.prep_coop_only) return n;
    for (int lv = 0; lv <= maxd; ++lv) {
      const int take = coop_take(blob, lv, H, DK, args.sgrid);
      for (int k = 0; k < take; ++k) {
        const int sg = level_seg[level_off[lv] + k];
        const int nc = (seg_len[sg] + CH - 1) / CH;
        if (n < nc) return chunk_base[sg] + n;
        n -= nc;
      }
    }
    return 0;  // (unreachable: n < nchunks)
  };
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
    const int n = item / H, h = item - n * H;
    const int2 ck = chunks[chunk_of(n)];
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

  int par = 0;
  for (int item = blockIdx.x; item < nchunks * H; item += gridDim.x, par ^= 1) {
    const int n = item / H, h = item - n * H;
    const int c = chunk_of(n);
    unsigned char* wsb = args.ws + ((size_t)c * H + h) * kWsChunk;
    float* gs = gsb[par];
    float* bs = bsb[par];

    // ---- stage K and Q; wave 0: g = inclusive cumulative sum of log a
    // (padding rows: a = 1, b = 0)
    const int len = rlen;
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int task = tid + 256 * i, row = task / CPR, ch = task % CPR;
      *(u32x4_t*)(Ks + row * LDK + ch * G::EPC) = row < len ? rk[i] : z4;
      *(u32x4_t*)(Qs + row * LDK + ch * G::EPC) = row < len ? rq[i] : z4;
    }
    if (w == 0) {
      const float la = wave_incl_scan(lane < len ? log_gate(ra) : 0.f, lane);
      gs[lane] = la;
      bs[lane] = lane < len ? rb : 0.f;
      if constexpr (BF16) {
        const float gl = lane_val(la, CH - 1);
        ((float*)(wsb + kWsGam))[lane] = __expf(la);
        ((float*)(wsb + kWsGam))[CH + lane] = __expf(gl - la);
      } else {
        ((float*)(wsb + 2 * kWsPlane))[lane] = la;
      }
    }
    if (item + (int)gridDim.x < nchunks * H) prep_load(item + gridDim.x);
    lds_barrier();  // K, Q, g and b are staged

    // ---- products Pt_J = K_J Q_w^T, At_J = K_J K_w^T (J <= w)
    f32x4_t pt[4], at[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) pt[J] = at[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      typename G::F bq[NKS], bk[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bq[ks] = ld_rowk<BF16>(Qs, LDK, 16 * w + c16, ks * G::KSTEP, q4);
        bk[ks] = ld_rowk<BF16>(Ks, LDK, 16 * w + c16, ks * G::KSTEP, q4);
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= w) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const typename G::F aK = ld_rowk<BF16>(Ks, LDK, 16 * J + c16, ks * G::KSTEP, q4);
            pt[J] = mma<BF16>(aK, bq[ks], pt[J]);
            at[J] = mma<BF16>(aK, bk[ks], at[J]);
          }
        }
      }
    }
    const int i = 16 * w + c16;  // this lane's row of P and A
    const float gi = gs[i], bi = bs[i];
    f32x4_t gj4[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) gj4[J] = *(const f32x4_t*)(gs + 16 * J + 4 * q4);
    lds_barrier();  // every wave is done reading Ks / Qs (A overwrites them)

    // ---- decays: P_ij = exp(g_i - g_j) (q_i . k_j) for j <= i, and
    // A_ij = b_i exp(g_i - g_j) (k_i . k_j) for j < i; A rows to LDS, P out
    f32x4_t pv[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      pv[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (J <= w) {
        f32x4_t av;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * J + 4 * q4 + r;
          const float dec = j <= i ? __expf(gi - gj4[J][r]) : 0.f;
          pv[J][r] = dec * pt[J][r];
          av[r] = j < i ? bi * dec * at[J][r] : 0.f;
        }
        *(f32x4_t*)(As + i * LDA + 16 * J + 4 * q4) = av;
      }
    }
    if constexpr (BF16) {
      u32x4_t* Pw = (u32x4_t*)(wsb + kWsFrag);
#pragma unroll
      for (int kf = 0; kf < 2; ++kf) {
        if (kf < frag_nk(w)) {
          const int fb = frag_tri(w) + kf;
          u32x2_t h0, l0, h1, l1;
          split4(pv[2 * kf], h0, l0);
          split4(pv[2 * kf + 1], h1, l1);
          Pw[(2 * fb) * 64 + lane] = u32x4_t{h0.x, h0.y, h1.x, h1.y};
          Pw[(2 * fb + 1) * 64 + lane] = u32x4_t{l0.x, l0.y, l1.x, l1.y};
        }
      }
    } else {
      float* Pw = (float*)(wsb + kWsPlane);
#pragma unroll
      for (int J = 0; J < 4; ++J) *(f32x4_t*)(Pw + i * CH + 16 * J + 4 * q4) = pv[J];
    }

    // ---- diagonal blocks of T (wave w: block w; its rows of A are its own stores)
    diag_inverse(As, Ts, LDA, 16 * w, lane);
    lds_barrier();

    // ---- blocks below the diagonal, by distance d = I - J (wave w: J = w).
    // Z = sum_K A_IK T_KJ comes out of the MFMA in accumulator order (lane
    // (c16, q4) holds Z[4 q4 + r][c16]), which is the B operand of T_II Z when
    // the reduction index of step r is 4 q4 + r; T_II is read in that order.
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int I = w + d, J = w;
      if (I < 4) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        for (int Kb = J; Kb < I; ++Kb) {
          const f32x4_t a4 = *(const f32x4_t*)(As + (16 * I + c16) * LDA + 16 * Kb + 4 * q4);
#pragma unroll
          for (int r = 0; r < 4; ++r) z = mma_f32(a4[r], Ts[(16 * Kb + 4 * q4 + r) * LDA + 16 * J + c16], z);
        }
        const f32x4_t t4 = *(const f32x4_t*)(Ts + (16 * I + c16) * LDA + 16 * I + 4 * q4);
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) t = mma_f32(t4[r], z[r], t);
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[(16 * I + 4 * q4 + r) * LDA + 16 * J + c16] = -t[r];
      }
      lds_barrier();
    }

    // ---- T'' = T diag(b) (zero above the diagonal) -> workspace
    if constexpr (BF16) {
      // operand fragments, hi and lo planes, one 16-byte group per task
      for (int task = tid; task < kNtri * 64; task += 256) {
        const int fb = task >> 6, l = task & 63;
        const int I = fb < 3 ? fb : (fb == 3 ? 2 : 3), kf = fb - frag_tri(I);
        const int ti = 16 * I + (l & 15), j0 = 32 * kf + 4 * (l >> 4);
        f32x4_t t0, t1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t0[e] = j0 + e <= ti ? Ts[ti * LDA + j0 + e] * bs[j0 + e] : 0.f;
          t1[e] = j0 + 16 + e <= ti ? Ts[ti * LDA + j0 + 16 + e] * bs[j0 + 16 + e] : 0.f;
        }
        u32x2_t h0, l0, h1, l1;
        split4(t0, h0, l0);
        split4(t1, h1, l1);
        u32x4_t* Tw = (u32x4_t*)wsb;
        Tw[(2 * fb) * 64 + l] = u32x4_t{h0.x, h0.y, h1.x, h1.y};
        Tw[(2 * fb + 1) * 64 + l] = u32x4_t{l0.x, l0.y, l1.x, l1.y};
      }
    } else {
      // row-major fp32 plane, 8 consecutive elements of a row per task
#pragma unroll
      for (int k = 0; k < CH * CH / 8 / 256; ++k) {
        const int idx8 = tid + 256 * k, ti = idx8 >> 3, j0 = (idx8 & 7) * 8;
        float tv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tv[e] = j0 + e <= ti ? Ts[ti * LDA + j0 + e] * bs[j0 + e] : 0.f;
        float* Tw = (float*)wsb + (size_t)ti * CH + j0;
        *(f32x4_t*)Tw = f32x4_t{tv[0], tv[1], tv[2], tv[3]};
        *(f32x4_t*)(Tw + 4) = f32x4_t{tv[4], tv[5], tv[6], tv[7]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Scan: one launch per tree depth. A work item is (segment, head, group of
// NSW 16-row slices of the state). Rows of the state evolve independently, so
// slices never communicate: one wave owns one slice and processes all 64 rows
// of every chunk for it. The chunk operands (k, q, T'', P, v, the decays) are
// loaded once per workgroup, coalesced, into LDS and shared by its waves.
//
// Register-resident chain. Every product is a 16x16 MFMA whose reduction index
// is enumerated in the order in which an accumulator already holds it: a
// 16x16 accumulator block gives lane (col c, group q) the rows 4q..4q+3, so a
// reduction step over 32 indices takes blocks 2f and 2f+1 and lane group q
// covers indices 32f + 4q + {0..3} and 32f + 16 + 4q + {0..3}. Operands read
// from LDS use the same order (two 8-byte reads per fragment, or two LDS
// transpose reads for a transposed operand). So the state S (held as S^T
// blocks), R = V - gamma X, U and U' pass from one product to the next in
// registers: no exchange through memory and no synchronisation inside a chunk.
//   X   = K S^T            (rows i, cols e)   A = K from LDS, B = S from regs
//   Y^T = S Q^T            (rows e, cols i)   A = S regs,     B = Q from LDS
//   U   = T'' R            (rows i, cols e)   A = T'' LDS,    B = R regs
//   Z^T = U^T P^T          (rows e, cols i)   A = U regs,     B = P LDS
//   S^T = gamma_C S^T + K^T U'  (rows d, cols e)  A = K^T (LDS transpose), B = U'
// fp32 mode uses the 16x16x4 fp32 MFMA with the same index order (step f is
// block f / 4, register f % 4).
template <bool BF16, int DK>
struct ScanCfg {
  using G = GT<BF16>;
  static constexpr int DV = DK;
  static constexpr int NSW = (BF16 ? 4 : 2) < DV / 16 ? (BF16 ? 4 : 2) : DV / 16;  // slices per workgroup
  static constexpr int NT = 64 * NSW;           // threads (one wave per slice)
  static constexpr int NG = DV / (16 * NSW);    // slice groups per head
  // Padded row lengths of the LDS tiles (elements), chosen from measured LDS
  // bank conflicts on gfx950 (the bank pattern repeats every 64 bf16): rows
  // of 4 or 12 (mod 64) make the 16-row fragment reads (ld_perm) conflict-free,
  // rows of 16 (mod 64) the transpose reads; K (read both ways) uses 12, which
  // leaves the transpose reads nearly free. Rows that are not a multiple of 16
  // bytes are staged with 8-byte stores.
  static constexpr int LDK = DK + (BF16 ? 12 : G::PAD);   // K, Q tiles
  static constexpr int LDT = CH + (BF16 ? 4 : G::PAD);    // T'', P tiles
  static constexpr int VW = 16 * NSW;                     // v columns of the group
  static constexpr int LDV = VW + (BF16 ? 16 : G::PAD);
  static constexpr int NDB = DK / 16;           // 16-wide d blocks of the state
  static constexpr int NKD = DK / G::KSTEP;     // reduction steps over d
  static constexpr int NKI = CH / G::KSTEP;     // reduction steps over chunk rows
  // reduction steps of the lower-triangular products for output row block I,
  // and the total over the four row blocks
  static constexpr int nk(int I) { return (16 * (I + 1) + G::KSTEP - 1) / G::KSTEP; }
  static constexpr int tri(int I) { return I == 0 ? 0 : tri(I - 1) + nk(I - 1); }
  static constexpr int NTRI = tri(4);
  // 16-byte chunks per thread of each staged operand
  static constexpr int KCH = CH * (DK / G::EPC) / NT;
  // T'' and P: bf16 fragments (hi, lo) as the prep kernel wrote them; fp32 planes
  static constexpr int TPB = BF16 ? (int)kWsFrag : (int)kWsPlane;  // bytes of T'' (and of P)
  static constexpr int WCH = TPB / 16 / NT;
  static constexpr int VCH = CH * (VW / G::EPC) / NT;
  static_assert(KCH * NT == CH * (DK / G::EPC), "K/Q staging must divide evenly");
  static_assert(WCH * NT * 16 == TPB, "T''/P staging must divide evenly");
  static_assert(VCH * NT == CH * (VW / G::EPC), "V staging must divide evenly");
  // LDS elements of one buffer's tiles; two buffers when they fit
  static constexpr int SK = CH * LDK, ST = CH * LDT, SV = CH * LDV;
  static constexpr int NPL = BF16 ? 2 : 1;  // planes of T'' and P (hi, lo)
  static constexpr size_t BUF_BYTES =
      (size_t)(2 * SK + SV) * sizeof(typename G::E) + (BF16 ? 2 * TPB : 2 * ST * 4) + 2 * CH * 4;
  static constexpr int NBUF = 2 * BUF_BYTES <= 160 * 1024 ? 2 : 1;
};

// Element offset of (row r, column col) in a row-major LDS tile with rows of
// W elements (padded, so that the reads below spread over the LDS banks).
template <bool BF16, int W>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * W + col;
}
// Stores one 16-byte group (8 bf16 / 4 fp32 elements starting at column col);
// as two 8-byte stores when rows are not 16-byte aligned.
template <bool BF16, int W>
__device__ __forceinline__ void tile_put16(typename GT<BF16>::E* tile, int r, int col, u32x4_t v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr ((W * sizeof(typename GT<BF16>::E)) % 16 == 0) {
    *(u32x4_t*)(tile + r * W + col) = v;
  } else {
    constexpr int HALF = 8 / sizeof(typename GT<BF16>::E);
    *(u32x2*)(tile + r * W + col) = u32x2{v.x, v.y};
    *(u32x2*)(tile + r * W + col + HALF) = u32x2{v.z, v.w};
  }
}

template <bool BF16, int DK>
struct ScanPrefetch {
  using C = ScanCfg<BF16, DK>;
  u32x4_t k[C::KCH], q[C::KCH], t[C::WCH], p[C::WCH], v[C::VCH];
  float g, gl;
};

// Global loads of chunk (t0, len) for head h and v columns [ve0, ve0 + VW),
// in two parts (k, q; then T'', P, v, g) so their issue spreads over the
// previous chunk's compute. Rows past len are clamped to the chunk's last row:
// they only meet zero coefficients (b = 0 there, so T'' has zero rows and
// columns and U zero rows) or produce output rows that are never stored, so
// no load needs a divergent branch.
template <bool BF16, int DK>
__device__ __forceinline__ void prefetch_kq(ScanPrefetch<BF16, DK>& r, const typename GT<BF16>::E* __restrict__ Kg,
                                            const typename GT<BF16>::E* __restrict__ Qg, int t0, int len, int H,
                                            int h, int tid) {
  using G = GT<BF16>;
  using C = ScanCfg<BF16, DK>;
  constexpr int CPR = DK / G::EPC;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int task = tid + C::NT * i, row = min(task / CPR, len - 1), ch = task % CPR;
    const size_t off = ((size_t)(t0 + row) * H + h) * DK + ch * G::EPC;
    r.k[i] = *(const u32x4_t*)(Kg + off);
    r.q[i] = *(const u32x4_t*)(Qg + off);
  }
}
template <bool BF16, int DK>
__device__ __forceinline__ void prefetch_rest(ScanPrefetch<BF16, DK>& r, const typename GT<BF16>::E* __restrict__ Vg,
                                              const unsigned char* __restrict__ wsb, int t0, int len, int H, int h,
                                              int ve0, int tid) {
  using G = GT<BF16>;
  using C = ScanCfg<BF16, DK>;
  const u32x4_t* Tw = (const u32x4_t*)wsb;
  const u32x4_t* Pw = (const u32x4_t*)(wsb + C::TPB);
#pragma unroll
  for (int i = 0; i < C::WCH; ++i) {
    r.t[i] = Tw[tid + C::NT * i];
    r.p[i] = Pw[tid + C::NT * i];
  }
  constexpr int VCPR = C::VW / G::EPC;
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int task = tid + C::NT * i;
    const int row = min(task / VCPR, len - 1), ch = task % VCPR;
    r.v[i] = *(const u32x4_t*)(Vg + ((size_t)(t0 + row) * H + h) * C::DV + ve0 + ch * G::EPC);
  }
  if constexpr (BF16) {
    // gamma and gamma_C / gamma
    const float* gw = (const float*)(wsb + kWsGam);
    r.g = gw[tid & (CH - 1)];
    r.gl = gw[CH + (tid & (CH - 1))];
  } else {
    // g; the decays are formed at staging
    const float* gw = (const float*)(wsb + 2 * kWsPlane);
    r.g = gw[tid & (CH - 1)];
    r.gl = gw[CH - 1];
  }
}

// One LDS buffer of chunk tiles.
template <bool BF16, int DK>
struct ScanTiles {
  using E = typename GT<BF16>::E;
  using C = ScanCfg<BF16, DK>;
  E* K;
  E* Q;
  E* Th;  // fp32: row-major T'' and P tiles; bf16: their fragments (hi, lo)
  E* Ph;
  E* V;
  float* gam;
  float* rr;
  __device__ __forceinline__ ScanTiles(unsigned char* base) {
    E* e = (E*)base;
    K = e;
    Q = e + C::SK;
    V = e + 2 * C::SK;
    unsigned char* tp = (unsigned char*)(V + C::SV);
    Th = (E*)tp;
    Ph = (E*)(tp + (BF16 ? C::TPB : C::ST * 4));
    gam = (float*)(tp + (BF16 ? 2 * C::TPB : 2 * C::ST * 4));
    rr = gam + CH;
  }
};

template <bool BF16, int DK>
__device__ __forceinline__ void stage_kq(const ScanTiles<BF16, DK>& b, const ScanPrefetch<BF16, DK>& r, int tid) {
  using G = GT<BF16>;
  using C = ScanCfg<BF16, DK>;
  constexpr int CPR = DK / G::EPC;
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int task = tid + C::NT * i, row = task / CPR, ch = task % CPR;
    tile_put16<BF16, C::LDK>(b.K, row, ch * G::EPC, r.k[i]);
    tile_put16<BF16, C::LDK>(b.Q, row, ch * G::EPC, r.q[i]);
  }
}
template <bool BF16, int DK>
__device__ __forceinline__ void stage_rest(const ScanTiles<BF16, DK>& b, const ScanPrefetch<BF16, DK>& r, int tid) {
  using G = GT<BF16>;
  using C = ScanCfg<BF16, DK>;
#pragma unroll
  for (int i = 0; i < C::WCH; ++i) {
    const int cidx = tid + C::NT * i;  // 16-byte chunk of the operand region
    if constexpr (BF16) {
      ((u32x4_t*)b.Th)[cidx] = r.t[i];
      ((u32x4_t*)b.Ph)[cidx] = r.p[i];
    } else {
      tile_put16<BF16, C::LDT>(b.Th, cidx / 16, (cidx % 16) * 4, r.t[i]);
      tile_put16<BF16, C::LDT>(b.Ph, cidx / 16, (cidx % 16) * 4, r.p[i]);
    }
  }
  constexpr int VCPR = C::VW / G::EPC;
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int task = tid + C::NT * i;
    tile_put16<BF16, C::LDV>(b.V, task / VCPR, (task % VCPR) * G::EPC, r.v[i]);
  }
  if (tid < CH) {
    if constexpr (BF16) {
      b.gam[tid] = r.g;
      b.rr[tid] = r.gl;
    } else {
      b.gam[tid] = __expf(r.g);
      b.rr[tid] = __expf(r.gl - r.g);
    }
  }
}

// Reduction step f of accumulator blocks X[] as an operand fragment (hi part,
// and in bf16 mode the lo part x - hi). Values are converted in pairs: one
// packed conversion gives both hi halves, whose float values are the packed
// word shifted / masked, so a pair costs 6 VALU operations.
template <bool BF16>
__device__ __forceinline__ void reg_frag(const f32x4_t* X, int f, typename GT<BF16>::F& hi,
                                         typename GT<BF16>::F& lo) {
  if constexpr (BF16) {
    u32x4_t h, l;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float a = X[2 * f + (p >> 1)][2 * (p & 1)], b = X[2 * f + (p >> 1)][2 * (p & 1) + 1];
      const unsigned w = pack_bf16x2(a, b);
      h[p] = w;
      l[p] = pack_bf16x2(a - __uint_as_float(w << 16), b - __uint_as_float(w & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8_t, h);
    lo = __builtin_bit_cast(bf16x8_t, l);
  } else {
    hi = X[f >> 2][f & 3];
    lo = 0.f;
  }
}

// Operand fragment of a row-major LDS matrix M[row][k] at reduction step f in
// the accumulator index order.
template <bool BF16, int W>
__device__ __forceinline__ typename GT<BF16>::F ld_perm(const typename GT<BF16>::E* base, int row, int f, int q4) {
  if constexpr (BF16) {
    const u32x2_t a = *(const u32x2_t*)(base + tile_off<BF16, W>(row, 32 * f + 4 * q4));
    const u32x2_t b = *(const u32x2_t*)(base + tile_off<BF16, W>(row, 32 * f + 16 + 4 * q4));
    const u32x4_t v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, v);
  } else {
    return base[tile_off<BF16, W>(row, 16 * (f >> 2) + 4 * q4 + (f & 3))];
  }
}

// Operand fragment of the transpose of a row-major LDS matrix M[k][col]
// (row of the fragment = column col0 + lane % 16 of M), step f in the
// accumulator index order. bf16: LDS transpose reads; within each 16-lane
// group lane m supplies row kb + m / 4, column col0 + 4 (m % 4), and lane i
// receives rows kb .. kb + 3 of column col0 + i.
template <bool BF16, int W>
__device__ __forceinline__ typename GT<BF16>::F ld_perm_t(const typename GT<BF16>::E* base, int col0, int f,
                                                          int lane) {
  const int q4 = lane >> 4, m = lane & 15;
  if constexpr (BF16) {
    const int r0 = 32 * f + 4 * q4 + (m >> 2), col = col0 + 4 * (m & 3);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + tile_off<BF16, W>(r0, col)));
    const s16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + tile_off<BF16, W>(r0 + 16, col)));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    return base[tile_off<BF16, W>(16 * (f >> 2) + 4 * q4 + (f & 3), col0 + m)];
  }
}

// Keeps the scheduler from moving instructions across this point, so LDS
// reads issued for the next group of products stay ahead of the current
// group's MFMAs (with one wave per SIMD nothing else hides their latency).
#define SCAN_FENCE() __builtin_amdgcn_sched_barrier(0)

template <bool BF16, int DK>
__global__ void __launch_bounds__((ScanCfg<BF16, DK>::NT)) gdn_scan_kernel(const int32_t* __restrict__ blob,
                                                                        GdnArgs args) {
  using G = GT<BF16>;
  using E = typename G::E;
  using F = typename G::F;
  using C = ScanCfg<BF16, DK>;
  using PF = ScanPrefetch<BF16, DK>;
  using TL = ScanTiles<BF16, DK>;
  constexpr bool SPLIT = BF16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::NBUF * C::BUF_BYTES];

  if (!blob_ok(blob, args.guard)) return;
  const int level = args.level;
  const bool planned = args.lv_first >= 0;
  if (!planned && level > blob[MH_MAXDEPTH]) return;
  const int32_t* __restrict__ level_off = blob + blob[MH_OFF_LEVELOFF];
  const int32_t* __restrict__ level_seg = blob + blob[MH_OFF_LEVELSEG];
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ root_ord = blob + blob[MH_OFF_ROOTORD];
  const int32_t* __restrict__ first_child = blob + blob[MH_OFF_FIRSTCHILD];
  const int32_t* __restrict__ chunk_base = blob + blob[MH_OFF_CHUNKBASE];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int H = args.H;
  // the depth's first `take` segments are handled by gdn_coop_kernel
  const int take = planned ? args.lv_take : (BF16 ? coop_segments(blob, level, H, C::DV) : 0);
  const int lv0 = (planned ? args.lv_first : level_off[level]) + take;
  const int nlev = (planned ? args.lv_first + args.lv_count : level_off[level + 1]) - lv0;
  const int tid = threadIdx.x, lane = tid & 63, sw = tid >> 6;  // wave = slice within the group
  const int c16 = lane & 15, q4 = lane >> 4;
  const E* __restrict__ Kg = (const E*)args.k;
  const E* __restrict__ Qg = (const E*)args.q;
  const E* __restrict__ Vg = (const E*)args.v;
  E* __restrict__ Og = (E*)args.o;
  const size_t SZ = (size_t)C::DV * DK;

  // Workgroups are dispatched round-robin over the 8 XCDs (workgroup id mod 8;
  // the grid is a multiple of 8), so item i runs on XCD i mod 8. Heads are
  // assigned so that all slice groups of one head share an XCD and its L2.
  const int NH8 = (H + 7) / 8;
  const int nitems = nlev * NH8 * 8 * C::NG;
  // work item -> (segment, head, slice group); uniform (scalar loads)
  struct ItemRef {
    int item, s, h, sg, L, st, cb;
  };
  auto find_item = [&](int from) {
    ItemRef r;
    r.item = nitems;
    for (int it = from; it < nitems; it += gridDim.x) {
      const int x = it & 7, j = it >> 3, j2 = j / C::NG;
      const int h = (j2 % NH8) * 8 + x;
      if (h >= H) continue;
      r.item = it;
      r.sg = j % C::NG;
      r.h = h;
      r.s = __builtin_amdgcn_readfirstlane(level_seg[lv0 + j2 / NH8]);
      r.L = __builtin_amdgcn_readfirstlane(seg_len[r.s]);
      r.st = __builtin_amdgcn_readfirstlane(seg_start[r.s]);
      r.cb = __builtin_amdgcn_readfirstlane(chunk_base[r.s]);
      break;
    }
    return r;
  };
  // The first chunk of the workgroup's next item is prefetched during the
  // current item's last chunk, so only the first item waits for its loads.
  PF nx;
  ItemRef cur = find_item(blockIdx.x);
  if (cur.item < nitems) {
    prefetch_kq<BF16, DK>(nx, Kg, Qg, cur.st, min(CH, cur.L), H, cur.h, tid);
    prefetch_rest<BF16, DK>(nx, Vg, args.ws + ((size_t)cur.cb * H + cur.h) * kWsChunk, cur.st, min(CH, cur.L), H,
                            cur.h, C::VW * cur.sg, tid);
  }
  for (; cur.item < nitems;) {
    const ItemRef nxi = find_item(cur.item + gridDim.x);
    const int sg = cur.sg, h = cur.h, s = cur.s, L = cur.L, st = cur.st, cb = cur.cb;
    // per-item metadata, uniform across the workgroup (scalar loads)
    const int p = __builtin_amdgcn_readfirstlane(parent[s]);
    const int fc_p = p >= 0 ? __builtin_amdgcn_readfirstlane(first_child[p]) : -1;
    const int ro = p < 0 ? __builtin_amdgcn_readfirstlane(root_ord[s]) : 0;
    const int ve0 = C::VW * sg;    // first v column (state row) of the group
    const int e0 = ve0 + 16 * sw;  // first state row of this wave's slice
    // chunk ci of the segment covers tokens [st + 64 ci, st + min(64 (ci + 1), L))
    const int nck = (L + CH - 1) / CH;

    // ---- start state: root_state / zero, or the parent's end state (read from
    // the first child's start slot, where the parent's scan left it).
    // St[db]: lane (c16, q4) holds S[e0 + c16][16 db + 4 q4 + r], r = 0..3.
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
    const bool has_src = src != nullptr;
    const float* lsrc = has_src ? src : own_slot;  // always a valid address
    const size_t srow = (size_t)(e0 + c16) * DK + 4 * q4;
    f32x4_t St[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const f32x4_t xv = *(const f32x4_t*)(lsrc + srow + 16 * db);
      St[db] = has_src ? xv : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (dst) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) *(f32x4_t*)(dst + srow + 16 * db) = St[db];
    }
    if constexpr (C::NBUF == 2) {
      __syncthreads();  // the previous item's last chunk no longer reads buffer 0
      const TL b0(lds);
      stage_kq<BF16, DK>(b0, nx, tid);
      stage_rest<BF16, DK>(b0, nx, tid);
    }

    // output tile of the previous chunk (O^T blocks: lane (c16, q4) holds
    // O[16 I + c16][e0 + 4 q4 + r]), stored one chunk late, after the next
    // chunk's loads are issued (a load issued after a possibly aliasing store
    // waits for that store)
    f32x4_t oval[4];
    int orow0 = 0, olen = 0;
    auto flush_o = [&]() {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int i = 16 * I + c16;
        if (i < olen) {
          E* d = Og + ((size_t)(orow0 + i) * H + h) * C::DV + e0 + 4 * q4;
          if constexpr (BF16) {
            const u32x2_t pk = {(unsigned)bf16_bits(oval[I][0]) | ((unsigned)bf16_bits(oval[I][1]) << 16),
                                (unsigned)bf16_bits(oval[I][2]) | ((unsigned)bf16_bits(oval[I][3]) << 16)};
            *(u32x2_t*)d = pk;
          } else {
            *(f32x4_t*)d = oval[I];
          }
        }
      }
    };

    for (int ci = 0; ci < nck; ++ci) {
      const int c = cb + ci;
      const int t0 = st + CH * ci, len = min(CH, L - CH * ci);
      const bool more = ci + 1 < nck;
      const int nt0 = t0 + CH, nlen = min(CH, L - CH * (ci + 1));
      const unsigned char* nws = args.ws + ((size_t)(c + 1) * H + h) * kWsChunk;
      const int bi = C::NBUF == 2 ? (ci & 1) : 0;
      const TL cur(lds + bi * C::BUF_BYTES);
      const TL nxt(lds + (C::NBUF == 2 ? (bi ^ 1) : 0) * C::BUF_BYTES);

      __syncthreads();  // this chunk's tiles are complete; the other buffer is free
      if constexpr (C::NBUF == 1) {
        stage_kq<BF16, DK>(cur, nx, tid);
        stage_rest<BF16, DK>(cur, nx, tid);
        __syncthreads();
      }
      if (more)
        prefetch_kq<BF16, DK>(nx, Kg, Qg, nt0, nlen, H, h, tid);
      else if (nxi.item < nitems)
        prefetch_kq<BF16, DK>(nx, Kg, Qg, nxi.st, min(CH, nxi.L), H, nxi.h, tid);

      // (1) X = K S^T and Y^T = S Q^T, LDS reads one reduction step ahead
      f32x4_t X[4], Yt[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) X[I] = Yt[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      F ka[2][4], qb[2][4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        ka[0][I] = ld_perm<BF16, C::LDK>(cur.K, 16 * I + c16, 0, q4);
        qb[0][I] = ld_perm<BF16, C::LDK>(cur.Q, 16 * I + c16, 0, q4);
      }
      F th[C::NTRI], tl[C::NTRI];
      f32x4_t vq[4], gq[4];
#pragma unroll
      for (int f = 0; f < C::NKD; ++f) {
        if (f + 1 < C::NKD) {
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            ka[(f + 1) & 1][I] = ld_perm<BF16, C::LDK>(cur.K, 16 * I + c16, f + 1, q4);
            qb[(f + 1) & 1][I] = ld_perm<BF16, C::LDK>(cur.Q, 16 * I + c16, f + 1, q4);
          }
        } else {
          // operands of steps (2) and (3)
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            if constexpr (BF16) {
              const unsigned short* pv =
                  cur.V + tile_off<BF16, C::LDV>(16 * I + 4 * q4 + (c16 >> 2), 16 * sw + 4 * (c16 & 3));
              const s16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)pv);
#pragma unroll
              for (int r = 0; r < 4; ++r) vq[I][r] = bf16_val((unsigned short)t[r]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) vq[I][r] = cur.V[tile_off<BF16, C::LDV>(16 * I + 4 * q4 + r, 16 * sw + c16)];
            }
            gq[I] = *(const f32x4_t*)(cur.gam + 16 * I + 4 * q4);
          }
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int kf = 0; kf < C::nk(I); ++kf) {
              if constexpr (BF16) {
                const u32x4_t* tf = (const u32x4_t*)cur.Th + (C::tri(I) + kf) * 128 + lane;
                th[C::tri(I) + kf] = __builtin_bit_cast(bf16x8_t, tf[0]);
                tl[C::tri(I) + kf] = __builtin_bit_cast(bf16x8_t, tf[64]);
              } else {
                th[C::tri(I) + kf] = ld_perm<BF16, C::LDT>(cur.Th, 16 * I + c16, kf, q4);
              }
            }
        }
        SCAN_FENCE();
        F sh, sl;
        reg_frag<BF16>(St, f, sh, sl);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          X[I] = mma<BF16>(ka[f & 1][I], sh, X[I]);
          Yt[I] = mma<BF16>(sh, qb[f & 1][I], Yt[I]);
          if constexpr (SPLIT) {
            X[I] = mma<BF16>(ka[f & 1][I], sl, X[I]);
            Yt[I] = mma<BF16>(sl, qb[f & 1][I], Yt[I]);
          }
        }
        SCAN_FENCE();
      }
      if (more)
        prefetch_rest<BF16, DK>(nx, Vg, nws, nt0, nlen, H, h, ve0, tid);
      else if (nxi.item < nitems)
        prefetch_rest<BF16, DK>(nx, Vg, args.ws + ((size_t)nxi.cb * H + nxi.h) * kWsChunk, nxi.st, min(CH, nxi.L),
                                H, nxi.h, C::VW * nxi.sg, tid);
      flush_o();

      // (2) R = V - gamma X  (lane (c16, q4), block I holds rows 16 I + 4 q4 + r)
      f32x4_t R[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) R[I] = vq[I] - gq[I] * X[I];
      F rh[C::NKI], rl[C::NKI];
#pragma unroll
      for (int f = 0; f < C::NKI; ++f) reg_frag<BF16>(R, f, rh[f], rl[f]);
      // (3) U = T'' R  (T'' lower triangular: row block I needs indices < 16 (I + 1));
      // the P fragments of step (4) are read meanwhile
      F ph[C::NTRI], pl[C::NTRI];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int kf = 0; kf < C::nk(I); ++kf) {
          if constexpr (BF16) {
            const u32x4_t* pf = (const u32x4_t*)cur.Ph + (C::tri(I) + kf) * 128 + lane;
            ph[C::tri(I) + kf] = __builtin_bit_cast(bf16x8_t, pf[0]);
            pl[C::tri(I) + kf] = __builtin_bit_cast(bf16x8_t, pf[64]);
          } else {
            ph[C::tri(I) + kf] = ld_perm<BF16, C::LDT>(cur.Ph, 16 * I + c16, kf, q4);
          }
        }
      SCAN_FENCE();
      f32x4_t U[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        U[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < C::nk(I); ++kf) {
          U[I] = mma<BF16>(th[C::tri(I) + kf], rh[kf], U[I]);
          if constexpr (SPLIT) {
            U[I] = mma<BF16>(th[C::tri(I) + kf], rl[kf], U[I]);
            U[I] = mma<BF16>(tl[C::tri(I) + kf], rh[kf], U[I]);
          }
        }
      }
      SCAN_FENCE();
      // (4) O^T = scale (S Q^T * gamma + U^T P^T), stored one chunk late; the
      // first K^T fragments of step (5) and the decays are read meanwhile
      F uh[C::NKI], ul[C::NKI];
#pragma unroll
      for (int f = 0; f < C::NKI; ++f) reg_frag<BF16>(U, f, uh[f], ul[f]);
      F kt[2][C::NDB];
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) kt[0][db] = ld_perm_t<BF16, C::LDK>(cur.K, 16 * db, 0, lane);
      f32x4_t rq[4];
      float gi[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        rq[I] = *(const f32x4_t*)(cur.rr + 16 * I + 4 * q4);
        gi[I] = cur.gam[16 * I + c16];
      }
      const float gC = cur.gam[CH - 1];
      SCAN_FENCE();
      f32x4_t Zt[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        Zt[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < C::nk(I); ++kf) {
          Zt[I] = mma<BF16>(uh[kf], ph[C::tri(I) + kf], Zt[I]);
          if constexpr (SPLIT) {
            Zt[I] = mma<BF16>(ul[kf], ph[C::tri(I) + kf], Zt[I]);
            Zt[I] = mma<BF16>(uh[kf], pl[C::tri(I) + kf], Zt[I]);
          }
        }
      }
      SCAN_FENCE();
      if constexpr (C::NBUF == 2)
        if (more) stage_kq<BF16, DK>(nxt, nx, tid);
#pragma unroll
      for (int I = 0; I < 4; ++I) oval[I] = args.scale * (gi[I] * Yt[I] + Zt[I]);
      orow0 = t0;
      olen = len;
      // (5) S^T = gamma_C S^T + K^T U',  U' = diag(gamma_C / gamma) U
#pragma unroll
      for (int I = 0; I < 4; ++I) U[I] *= rq[I];
#pragma unroll
      for (int f = 0; f < C::NKI; ++f) reg_frag<BF16>(U, f, uh[f], ul[f]);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) St[db] *= gC;
#pragma unroll
      for (int f = 0; f < C::NKI; ++f) {
        if (f + 1 < C::NKI) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
            kt[(f + 1) & 1][db] = ld_perm_t<BF16, C::LDK>(cur.K, 16 * db, f + 1, lane);
        }
        SCAN_FENCE();
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          St[db] = mma<BF16>(kt[f & 1][db], uh[f], St[db]);
          if constexpr (SPLIT) St[db] = mma<BF16>(kt[f & 1][db], ul[f], St[db]);
        }
        SCAN_FENCE();
      }
      if constexpr (C::NBUF == 2)
        if (more) stage_rest<BF16, DK>(nxt, nx, tid);
    }
    flush_o();

    // ---- end state: seg_final_state and the first child's start slot (the fork)
    {
      const int fc = __builtin_amdgcn_readfirstlane(first_child[s]);
      float* d1 = args.seg_final ? args.seg_final + ((size_t)s * H + h) * SZ : nullptr;
      float* d2 = fc >= 0 ? args.seg_start + ((size_t)fc * H + h) * SZ : nullptr;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        if (d1) *(f32x4_t*)(d1 + srow + 16 * db) = St[db];
        if (d2) *(f32x4_t*)(d2 + srow + 16 * db) = St[db];
      }
    }
    cur = nxi;
  }
}

// ---------------------------------------------------------------------------
// bf16 scan, chunk-cooperative with helper waves. One launch per tree depth;
// a work item is (segment, head, 16-row slice of the state). Its chunks run
// on a workgroup of 2 NW waves, NW = DK / 32:
//   chain wave w owns state columns [32 w, 32 w + 32) (two 16x16 blocks of
//   S^T, the reduction step w of every product over d) and token blocks
//   w, w + NW, ... (16 rows of the chunk each); it runs the serial part:
//     (1) X = K S^T, R = V - gamma X         -> exchange (hi, lo)
//     (3) U = T'' R, U' = diag(gamma_C / gamma) U   -> exchange (hi, lo of both)
//     (5) S^T = gamma_C S^T + K^T U'         -> exchange (next chunk's S)
//   helper wave v loads the next task's operands into LDS and computes the
//   outputs of token blocks v, v + NW, ...:
//     (4) O^T = scale (S Q^T * gamma + U^T P^T).
// Three workgroup barriers per chunk separate the exchanges. Each product's
// reduction index runs in the order of a 16x16 accumulator (lane group q
// holds rows 4q..4q+3), as written by the exchanges and by the prep kernel's
// fragments; K and Q are read in the same order (two 8-byte reads, or two
// transposing reads for K^T).
// The operands of a chunk (K, Q, T'' and P fragments, the slice's v columns,
// the decays, and at a segment's first chunk its start state) are fetched by
// buffer loads straight into LDS, double-buffered: the next task (the next
// chunk, or the first chunk of the workgroup's next item) loads while the
// current one computes, its loads spread over the first two phases. The buffer
// range of K, Q and V ends at the chunk's last token, so rows past a ragged
// chunk read as zeros; a missing start state (a root without root_state) is
// an empty range and reads as zeros too.
template <int DK>
struct CoopCfg {
  static constexpr int NW = DK / 32;           // chain waves (and helper waves)
  static constexpr int NT = 128 * NW;
  static constexpr int TB = 4 / NW;            // token blocks per wave
  static constexpr int CPR = DK / 8;           // 16-byte chunks per K/Q row
  static constexpr int NKD = DK / 32;          // reduction steps over d
  static constexpr int KQ = CH * DK * 2;       // bytes of the K (or Q) tile
  static constexpr int FR = (int)kWsFrag;      // T'' (or P) fragments
  static constexpr int VB = CH * 16 * 2;       // v columns of the slice, 64 tokens
  static constexpr int GB = 1024;              // gamma, gamma_C / gamma (one 1 KB load)
  static constexpr int SB = 16 * DK * 4;       // start state of the slice (fp32)
  static constexpr int OQ = KQ, OT = 2 * KQ, OP = OT + FR, OV = OP + FR, OG = OV + VB, OS = OG + GB;
  static constexpr int BUF = OS + SB;
  static constexpr int KJ = KQ / 1024;         // 1 KB loads of K (and of Q)
  static constexpr int FJ = FR / 1024;         // of T'' (and of P)
  static constexpr int SJ = SB / 1024;         // of the start state
  static_assert(KJ / NW == 4 && FJ % NW == 0 && SJ % NW == 0, "load split over the helper waves");
  static constexpr int XB = 2 * NKD * 64 * 16 + 2 * 4 * 64 * 8 + 4 * 4 * 64 * 8;  // exchanges
  static_assert(2 * BUF + XB <= 160 * 1024, "LDS");
};

// K/Q tiles in LDS: rows of DK bf16, unpadded; the 16-byte chunks of row r
// are permuted (chunk c at position c ^ kq_swz(r)) against conflicts on the 64
// banks of 4 bytes (one cycle serves 16 lanes of a 16-byte read, 32 of an
// 8-byte one). Rows of 16 chunks: kq_swz(r) = 2 (r mod 8) + (r / 8 mod 2), so
// the row reads (16 rows at one chunk) take 16 different bank groups and the
// transposing reads (8 rows x 32 bytes per cycle) 8 different pair slots.
// Rows of 8 chunks: 2 (r mod 4) + (r / 4 mod 2).
__device__ __forceinline__ int kq_swz(int r, int cpr) {
  return cpr >= 16 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r & 3) << 1) | ((r >> 2) & 1)) & (cpr - 1));
}
template <int DK>
__device__ __forceinline__ int kq_off(int r, int col) {
  return r * DK + 8 * ((col >> 3) ^ kq_swz(r, DK / 8)) + (col & 7);
}
// Fragment of K (or Q) rows at reduction step f in accumulator order.
template <int DK>
__device__ __forceinline__ bf16x8_t kq_frag(const unsigned short* t, int row, int f, int q4) {
  const u32x2_t a = *(const u32x2_t*)(t + kq_off<DK>(row, 32 * f + 4 * q4));
  const u32x2_t b = *(const u32x2_t*)(t + kq_off<DK>(row, 32 * f + 16 + 4 * q4));
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
}
// Fragment of K^T (row = column col0 + lane % 16 of K) at step f: two LDS
// transposing reads; within each 16-lane group lane m supplies row kb + m / 4,
// column col0 + 4 (m % 4), and lane i receives rows kb .. kb + 3 of column col0 + i.
template <int DK>
__device__ __forceinline__ bf16x8_t kt_frag(const unsigned short* t, int col0, int f, int lane) {
  const int q4 = lane >> 4, m = lane & 15;
  const int r0 = 32 * f + 4 * q4 + (m >> 2), col = col0 + 4 * (m & 3);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(t + kq_off<DK>(r0, col)));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(t + kq_off<DK>(r0 + 16, col)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The start state of the slice in LDS: 16 rows of DK floats; the 16-byte
// chunks of row r are permuted (chunk c at position c ^ (r mod 8)) so that a
// read of one column group by 16 rows spreads over the banks.
template <int DK>
__device__ __forceinline__ f32x4_t st_read(const float* t, int r, int col) {
  return *(const f32x4_t*)(t + r * DK + 4 * ((col >> 2) ^ (r & 7)));
}
__device__ __forceinline__ bf16x8_t join_frag(u32x2_t a, u32x2_t b) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
}
__device__ __forceinline__ bf16x8_t join_or_zero(bool live, u32x2_t a, u32x2_t b) {
  const u32x4_t z4 = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, live ? u32x4_t{a.x, a.y, b.x, b.y} : z4);
}

// Raw buffer resource: 64-bit base, no stride, num_records bytes in range;
// dword 3 selects the 32-bit data format. Loads past num_records return zeros.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buf_rsrc(const void* base, int bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4_t{(int)(unsigned)a, (int)(unsigned)((a >> 32) & 0xffffu), bytes, 0x00020000};
}
// 16 bytes per lane from buffer r at voff + soff into LDS at lds_base + OFF
// + 16 * lane. Written as inline assembly so that the compiler does not track these loads:
// it would otherwise wait for them before unrelated LDS reads. Completion is
// awaited explicitly (vmcnt) before the barrier that publishes the buffer.
// The leading s_nop covers the SGPR-write-to-VMEM-read and M0-write-to-LDS-DMA
// wait states; M0 (the LDS address) is restored afterwards.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(unsigned long long)(lds_void_t*)p; }
template <int OFF>
__device__ __forceinline__ void load_lds16(i32x4_t r, unsigned lds_base, int voff, int soff) {
  unsigned saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %5\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(r),
        "s"(__builtin_amdgcn_readfirstlane(soff)), "n"(OFF)
      : "memory", "scc");
}

// One chunk of one work item, with what its loads and stores need (uniform
// across the workgroup).
struct CoopTask {
  int item, ci, nck;
  int sst, L;      // the segment's first token and length
  int h, e0, ws0;  // head, first state row of the slice, workspace block of the segment's first chunk
  int s;           // segment: end state to seg_final_state[s]
  int src;         // start state: seg_start_state slot src (>= 0), root_state[-2 - src], or zeros (-1)
  int own;         // copy of the start state into the segment's own slot (s), or -1
  int fc;          // end state also to the first child's start slot, or -1
  int valid;
  __device__ int t0() const { return sst + CH * ci; }
  __device__ int len() const { return min(CH, L - CH * ci); }
};

template <int DK>
__global__ void __launch_bounds__(CoopCfg<DK>::NT) gdn_coop_kernel(const int32_t* __restrict__ blob,
                                                                  GdnArgs args) {
  using C = CoopCfg<DK>;
  constexpr int DV = DK;
  constexpr int NG = DV / 16;  // slices per head
  typedef unsigned short E;
  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::BUF];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::BUF];
  __shared__ u32x4_t sx[2][C::NKD][64];  // state fragments (hi, lo) of each reduction step
  __shared__ u32x2_t rx[2][4][64];       // R blocks (hi, lo)
  __shared__ u32x2_t ux[4][4][64];       // U blocks (hi, lo), U' blocks (hi, lo)

  if (!blob_ok(blob, args.guard)) return;
  const int level = args.level;
  const bool planned = args.lv_first >= 0;
  if (!planned && level > blob[MH_MAXDEPTH]) return;
  const int32_t* __restrict__ level_off = blob + blob[MH_OFF_LEVELOFF];
  const int32_t* __restrict__ level_seg = blob + blob[MH_OFF_LEVELSEG];
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ root_ord = blob + blob[MH_OFF_ROOTORD];
  const int32_t* __restrict__ first_child = blob + blob[MH_OFF_FIRSTCHILD];
  const int32_t* __restrict__ chunk_base = blob + blob[MH_OFF_CHUNKBASE];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int H = args.H;
  const int lv0 = planned ? args.lv_first : level_off[level];
  const int nlev = planned ? args.lv_take : coop_segments(blob, level, H, DV);
  if (nlev == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wv < C::NW;
  const int w = chain ? wv : wv - C::NW;  // chain wave w, or helper wave w
  const int c16 = lane & 15, q4 = lane >> 4;
  const E* __restrict__ Kg = (const E*)args.k;
  const E* __restrict__ Qg = (const E*)args.q;
  const E* __restrict__ Vg = (const E*)args.v;
  E* __restrict__ Og = (E*)args.o;
  const size_t SZ = (size_t)DV * DK;

  // Item i runs on XCD i mod 8 (workgroups are dispatched round-robin over
  // the 8 XCDs and the grid is a multiple of 8); all slices of a head share
  // an XCD and its L2.
  const int NH8 = (H + 7) / 8;
  const int nitems = nlev * NH8 * 8 * NG;
  // first chunk of the first valid item at or after `item` of this workgroup
  auto item_task = [&](int item) {
    CoopTask t;
    t.valid = 0;
    for (; item < nitems; item += gridDim.x) {
      const int x = item & 7, j = item >> 3;
      const int sg = j % NG, j2 = j / NG;
      const int h = (j2 % NH8) * 8 + x, li = j2 / NH8;
      if (h >= H) continue;
      const int s = __builtin_amdgcn_readfirstlane(level_seg[lv0 + li]);
      const int L = __builtin_amdgcn_readfirstlane(seg_len[s]);
      if (L <= 0) continue;
      const int p = __builtin_amdgcn_readfirstlane(parent[s]);
      t.item = item;
      t.ci = 0;
      t.nck = (L + CH - 1) / CH;
      t.sst = __builtin_amdgcn_readfirstlane(seg_start[s]);
      t.L = L;
      t.h = h;
      t.e0 = 16 * sg;
      t.ws0 = __builtin_amdgcn_readfirstlane(chunk_base[s]) * H + h;
      t.s = s;
      if (p < 0) {
        t.src = args.root_state ? -2 - __builtin_amdgcn_readfirstlane(root_ord[s]) : -1;
        t.own = s;
      } else {
        const int fc_p = __builtin_amdgcn_readfirstlane(first_child[p]);
        t.src = fc_p;
        t.own = fc_p != s ? s : -1;
      }
      t.fc = __builtin_amdgcn_readfirstlane(first_child[s]);
      t.valid = 1;
      break;
    }
    return t;
  };
  // the task after t: the segment's next chunk, or the next item's first
  auto next_task = [&](const CoopTask& t) {
    if (t.ci + 1 < t.nck) {
      CoopTask n = t;
      n.ci = t.ci + 1;
      return n;
    }
    return item_task(t.item + gridDim.x);
  };

  // ---- loads of a task's operands into LDS buffer b (helper waves), in two
  // parts spread over the first two phases of the current chunk: K, Q and (at
  // a segment's first chunk) the start state; T'', P, v and the decays
  auto dma = [&](unsigned char* b, const CoopTask& t, int part) {
    const int t0 = t.t0(), len = t.len();
    const unsigned lb = lds_addr(b) + 1024 * w;  // this wave's loads: 1 KB blocks w, w + NW, ...
    const i32x4_t rW = buf_rsrc(args.ws + (size_t)(t.ws0 + t.ci * H) * kWsChunk, (int)kWsChunk);
    // byte offset of this lane's 16 bytes in K/Q load i (rows past len are out of range)
    auto kvo = [&](int i) {
      const int n = 64 * (w + C::NW * i) + lane, r = n / C::CPR, c = (n % C::CPR) ^ kq_swz(r, C::CPR);
      return (r * H + t.h) * DK * 2 + 16 * c;
    };
    constexpr int S1 = 1024 * C::NW;  // stride of a wave's blocks
    if (part == 0) {
      const i32x4_t rK = buf_rsrc(Kg + (size_t)t0 * H * DK, len * H * DK * 2);
      const i32x4_t rQ = buf_rsrc(Qg + (size_t)t0 * H * DK, len * H * DK * 2);
      load_lds16<0 * S1>(rK, lb, kvo(0), 0);
      load_lds16<1 * S1>(rK, lb, kvo(1), 0);
      load_lds16<2 * S1>(rK, lb, kvo(2), 0);
      load_lds16<3 * S1>(rK, lb, kvo(3), 0);
      load_lds16<C::OQ + 0 * S1>(rQ, lb, kvo(0), 0);
      load_lds16<C::OQ + 1 * S1>(rQ, lb, kvo(1), 0);
      load_lds16<C::OQ + 2 * S1>(rQ, lb, kvo(2), 0);
      load_lds16<C::OQ + 3 * S1>(rQ, lb, kvo(3), 0);
      if (t.ci == 0) {
        // start state rows e0 .. e0 + 15 of DK floats; chunk c of row r at
        // position c ^ (r mod 8)
        const float* src = t.src >= 0 ? args.seg_start + ((size_t)t.src * H + t.h) * SZ
                           : t.src < -1 ? args.root_state + ((size_t)(-2 - t.src) * H + t.h) * SZ
                                        : args.seg_start;
        const i32x4_t rS = buf_rsrc(src + (size_t)t.e0 * DK, t.src != -1 ? C::SB : 0);
#pragma unroll
        for (int i = 0; i < C::SJ / C::NW; ++i) {
          const int n = 64 * (w + C::NW * i) + lane, r = n / (DK / 4), c = (n % (DK / 4)) ^ (r & 7);
          load_lds16<0>(rS, lb + C::OS + i * S1, r * DK * 4 + 16 * c, 0);
        }
      }
    } else {
      const int wo = 16 * lane + 1024 * w;
#pragma unroll
      for (int i = 0; i < C::FJ / C::NW; ++i) load_lds16<0>(rW, lb + C::OT + i * S1, wo, i * S1);
#pragma unroll
      for (int i = 0; i < C::FJ / C::NW; ++i) load_lds16<0>(rW, lb + C::OP + i * S1, wo, (int)kWsFrag + i * S1);
      if (w < 2 || C::NW == 1) {
        const i32x4_t rV = buf_rsrc(Vg + (size_t)t0 * H * DV, len * H * DV * 2);
        for (int jv = w; jv < 2; jv += C::NW) {
          const int n = 64 * jv + lane, r = n >> 1;
          load_lds16<C::OV>(rV, lds_addr(b) + 1024 * jv, (r * H + t.h) * DV * 2 + 2 * t.e0 + 16 * (n & 1), 0);
        }
      }
      if (w == C::NW - 1) load_lds16<C::OG>(rW, lds_addr(b), 16 * lane, (int)kWsGam);
    }
  };

  f32x4_t St[2];        // chain wave: S^T blocks, lane (c16, q4): S[e0 + c16][32 w + 16 jb + 4 q4 + r]
  f32x4_t oval[C::TB];  // helper wave: O^T blocks of the previous chunk, lane (c16, q4): O[16 I + c16][e0 + 4 q4 + r]
  int o_t0 = 0, o_len = 0, o_h = 0, o_e0 = 0;
  auto flush_o = [&]() {
#pragma unroll
    for (int bb = 0; bb < C::TB; ++bb) {
      const int i = 16 * (w + C::NW * bb) + c16;
      if (i < o_len) {
        E* d = Og + ((size_t)(o_t0 + i) * H + o_h) * DV + o_e0 + 4 * q4;
        *(u32x2_t*)d = u32x2_t{pack_bf16x2(oval[bb][0], oval[bb][1]), pack_bf16x2(oval[bb][2], oval[bb][3])};
      }
    }
    o_len = 0;
  };
  // S fragments of every reduction step: from the exchange, or at a
  // segment's first chunk from the start state in LDS
  auto s_frags = [&](const unsigned char* cb, bool first, bf16x8_t* sh, bf16x8_t* sl) {
#pragma unroll
    for (int f = 0; f < C::NKD; ++f) {
      if (first) {
        const float* S0 = (const float*)(cb + C::OS);
        u32x2_t ah, al, bh, bl;
        split4(st_read<DK>(S0, c16, 32 * f + 4 * q4), ah, al);
        split4(st_read<DK>(S0, c16, 32 * f + 16 + 4 * q4), bh, bl);
        sh[f] = join_frag(ah, bh);
        sl[f] = join_frag(al, bl);
      } else {
        sh[f] = __builtin_bit_cast(bf16x8_t, sx[0][f][lane]);
        sl[f] = __builtin_bit_cast(bf16x8_t, sx[1][f][lane]);
      }
    }
  };

  // One chunk (task c, operands in cur) while the next task's operands load
  // into nxt; n2 receives the task after that.
  auto step = [&](const unsigned char* cur, unsigned char* nxt, const CoopTask& c, const CoopTask& n1) {
    CoopTask n2;
    const E* Ks = (const E*)cur;
    const E* Qs = (const E*)(cur + C::OQ);
    const float* gam = (const float*)(cur + C::OG);
    const float* rrp = gam + CH;
    const bool first = c.ci == 0, last = c.ci + 1 == c.nck;
    if (!chain) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of the chunk landed
    lds_barrier();  // B0: the chunk's operands and S fragments are in LDS; nxt is no longer read
    f32x4_t Yt[C::TB];
    bf16x8_t th[C::TB][2], tl[C::TB][2], kt[2][2];
    f32x4_t rq[C::TB];
    if (chain) {
      // every LDS read of this phase first (one round trip), then the products;
      // T'' and the decays of phase (3) are read here too
      bf16x8_t sh[C::NKD], sl[C::NKD], ka[C::TB][C::NKD];
      s16x4_t vt[C::TB];
      f32x4_t gq[C::TB];
      s_frags(cur, first, sh, sl);
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb) {
        const int I = w + C::NW * bb;
#pragma unroll
        for (int f = 0; f < C::NKD; ++f) {
          ka[bb][f] = kq_frag<DK>(Ks, 16 * I + c16, f, q4);
        }
        vt[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)((const E*)(cur + C::OV) + (16 * I + 4 * q4 + (c16 >> 2)) * 16 + 4 * (c16 & 3)));
        gq[bb] = *(const f32x4_t*)(gam + 16 * I + 4 * q4);
        rq[bb] = *(const f32x4_t*)(rrp + 16 * I + 4 * q4);
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
          // T'' rows of block I < 2 have no second step: it reuses the first
          // fragment against zeros (below)
          const u32x4_t* tf = (const u32x4_t*)(cur + C::OT) + (frag_tri(I) + (kf < frag_nk(I) ? kf : 0)) * 128 + lane;
          th[bb][kf] = __builtin_bit_cast(bf16x8_t, tf[0]);
          tl[bb][kf] = __builtin_bit_cast(bf16x8_t, tf[64]);
        }
      }
      if (first) {
        const float* S0 = (const float*)(cur + C::OS);
        St[0] = st_read<DK>(S0, c16, 32 * w + 4 * q4);
        St[1] = st_read<DK>(S0, c16, 32 * w + 16 + 4 * q4);
      }
      SCAN_FENCE();
      // (1) X = K S^T, R = V - gamma X -> exchange
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb) {
        const int I = w + C::NW * bb;
        f32x4_t X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < C::NKD; ++f) {
          X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[bb][f], sh[f], X, 0, 0, 0);
          X = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[bb][f], sl[f], X, 0, 0, 0);
        }
        f32x4_t R;
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = bf16_val((unsigned short)vt[bb][r]) - gq[bb][r] * X[r];
        split4(R, rx[0][I][lane], rx[1][I][lane]);
      }
      if (first && c.own >= 0) {
        float* d = args.seg_start + ((size_t)c.own * H + c.h) * SZ + (size_t)(c.e0 + c16) * DK + 32 * w + 4 * q4;
        *(f32x4_t*)d = St[0];
        *(f32x4_t*)(d + 16) = St[1];
      }
    } else {
      if (n1.valid) {
        dma(nxt, n1, 0);
        dma(nxt, n1, 1);
      }
      flush_o();
    }
    lds_barrier();  // B1: R is exchanged
    if (chain) {
      // (3) U = T'' R, U' = diag(gamma_C / gamma) U -> exchange; the K^T
      // fragments of phase (5) are read with R
      bf16x8_t rh[2], rl[2];
#pragma unroll
      for (int kf = 0; kf < 2; ++kf) {
        rh[kf] = join_frag(rx[0][2 * kf][lane], rx[0][2 * kf + 1][lane]);
        rl[kf] = join_frag(rx[1][2 * kf][lane], rx[1][2 * kf + 1][lane]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) kt[kf][jb] = kt_frag<DK>(Ks, 32 * w + 16 * jb, kf, lane);
      }
      SCAN_FENCE();
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb) {
        const int I = w + C::NW * bb;
        f32x4_t U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
          const bool live = kf < frag_nk(I);
          const u32x4_t z4 = {0u, 0u, 0u, 0u};
          const bf16x8_t h = live ? rh[kf] : __builtin_bit_cast(bf16x8_t, z4);
          const bf16x8_t l = live ? rl[kf] : __builtin_bit_cast(bf16x8_t, z4);
          U = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th[bb][kf], h, U, 0, 0, 0);
          U = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th[bb][kf], l, U, 0, 0, 0);
          U = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl[bb][kf], h, U, 0, 0, 0);
        }
        split4(U, ux[0][I][lane], ux[1][I][lane]);
        split4(U * rq[bb], ux[2][I][lane], ux[3][I][lane]);
      }
    } else {
      // Y^T = S Q^T for this wave's token blocks (the chunk's S fragments stay
      // in the exchange, or at a segment's first chunk in the start state,
      // until the state update after B2)
      bf16x8_t sh[C::NKD], sl[C::NKD], qb[C::TB][C::NKD];
      s_frags(cur, first, sh, sl);
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb)
#pragma unroll
        for (int f = 0; f < C::NKD; ++f) qb[bb][f] = kq_frag<DK>(Qs, 16 * (w + C::NW * bb) + c16, f, q4);
      SCAN_FENCE();
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb) {
        Yt[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < C::NKD; ++f) {
          Yt[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sh[f], qb[bb][f], Yt[bb], 0, 0, 0);
          Yt[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl[f], qb[bb][f], Yt[bb], 0, 0, 0);
        }
      }
    }
    n2.valid = 0;
    if (n1.valid) n2 = next_task(n1);
    lds_barrier();  // B2: U and U' are exchanged
    if (chain) {
      // (5) S^T = gamma_C S^T + K^T U'; then the end state, or the next S fragments
      bf16x8_t uh[2], ul[2];
#pragma unroll
      for (int kf = 0; kf < 2; ++kf) {
        uh[kf] = join_frag(ux[2][2 * kf][lane], ux[2][2 * kf + 1][lane]);
        ul[kf] = join_frag(ux[3][2 * kf][lane], ux[3][2 * kf + 1][lane]);
      }
      const float gC = gam[CH - 1];
      St[0] *= gC;
      St[1] *= gC;
#pragma unroll
      for (int kf = 0; kf < 2; ++kf)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          St[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[kf][jb], uh[kf], St[jb], 0, 0, 0);
          St[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[kf][jb], ul[kf], St[jb], 0, 0, 0);
        }
      if (last) {
        const size_t srow = (size_t)(c.e0 + c16) * DK + 32 * w + 4 * q4;
        if (args.seg_final) {
          float* d = args.seg_final + ((size_t)c.s * H + c.h) * SZ + srow;
          *(f32x4_t*)d = St[0];
          *(f32x4_t*)(d + 16) = St[1];
        }
        if (c.fc >= 0) {
          float* d = args.seg_start + ((size_t)c.fc * H + c.h) * SZ + srow;
          *(f32x4_t*)d = St[0];
          *(f32x4_t*)(d + 16) = St[1];
        }
      } else {
        u32x2_t h0, l0, h1, l1;
        split4(St[0], h0, l0);
        split4(St[1], h1, l1);
        sx[0][w][lane] = u32x4_t{h0.x, h0.y, h1.x, h1.y};
        sx[1][w][lane] = u32x4_t{l0.x, l0.y, l1.x, l1.y};
      }
    } else {
      // (4) O^T = scale (gamma Y^T + U^T P^T), stored during the next chunk
#pragma unroll
      for (int bb = 0; bb < C::TB; ++bb) {
        const int I = w + C::NW * bb;
        f32x4_t Zt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
          const bool live = kf < frag_nk(I);
          const bf16x8_t uh = join_or_zero(live, ux[0][2 * kf][lane], ux[0][2 * kf + 1][lane]);
          const bf16x8_t ul = join_or_zero(live, ux[1][2 * kf][lane], ux[1][2 * kf + 1][lane]);
          const u32x4_t* pf = (const u32x4_t*)(cur + C::OP) + (frag_tri(I) + (live ? kf : 0)) * 128 + lane;
          const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, pf[0]);
          const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, pf[64]);
          Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh, ph, Zt, 0, 0, 0);
          Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul, ph, Zt, 0, 0, 0);
          Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh, pl, Zt, 0, 0, 0);
        }
        const float gi = gam[16 * I + c16];
        oval[bb] = args.scale * (gi * Yt[bb] + Zt);
      }
      o_t0 = c.t0();
      o_len = c.len();
      o_h = c.h;
      o_e0 = c.e0;
    }
    return n2;
  };

  CoopTask cur = item_task(blockIdx.x);
  if (!cur.valid) return;
  CoopTask n1 = next_task(cur);
  if (!chain) {
    dma(buf0, cur, 0);
    dma(buf0, cur, 1);
  }
  for (;;) {
    CoopTask n2 = step(buf0, buf1, cur, n1);
    if (!n1.valid) break;
    cur = n1;
    n1 = n2;
    n2 = step(buf1, buf0, cur, n1);
    if (!n1.valid) break;
    cur = n1;
    n1 = n2;
  }
  if (!chain) flush_o();
}

// ---------------------------------------------------------------------------
// Fused bf16 Gated DeltaNet (DK = DV = 128): chunk preparation and scan in one
// kernel, one work item = (segment, head) on one workgroup of 8 waves. Wave w
// owns state rows [16 w, 16 w + 16) (slices never communicate). Per chunk:
//   B0  the chunk's k, q, v, a, b are in LDS (this wave's loads waited, then
//       the barrier); the next chunk's loads (or the next item's first) are
//       issued into the other buffer;
//   prep (waves 0-3; wave 0 first forms the decays): Pt_J = K_J Q_w^T and
//       At_J = K_J K_w^T (J <= w) on MFMA, P = QK^T * Gamma as hi/lo operand
//       fragments and A = strictly_lower(diag(b) KK^T * Gamma) in LDS; the
//       diagonal blocks of T = (I + A)^-1 by forward substitution, the blocks
//       below by distance; T'' = T diag(b) as hi/lo fragments (all threads);
//   scan (every wave, its slice): X = K S^T, Y^T = S Q^T, R = V - gamma X,
//       U = T'' R, O^T = scale (gamma Y^T + U^T P^T), S^T = gamma_C S^T + K^T U'.
// So the chunk intermediates never leave the CU (no workspace round trip) and
// each chunk's operands are read once per head instead of once per group of
// slices. The start state comes from root_state / zero or the parent's end
// state (the parent's first child's start slot, where the parent's item left
// it) and is copied into the segment's own slot; the end state goes to
// seg_final_state and the first child's slot.
// FP8 code tiles in LDS: rows of DK = 128 bytes (8 chunks of 16 bytes, two
// rows per 256-byte bank cycle); chunk c of row r sits at position
// c ^ ((r / 2) mod 8), so the 16-byte reads of 16 consecutive rows at one
// chunk take 16 different bank groups. code8_chunk is its own inverse: the
// position of chunk c, and the chunk held at position c.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ int code8_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

struct FusedCfg {
  static constexpr int DK = 128, NW = 8, NT = 64 * NW;
  static constexpr int TB = CH * DK * 2;               // a K, Q or V tile (bf16, kq_off layout)
  static constexpr int OQ = TB, OV = 2 * TB, OA = 3 * TB, OB = OA + CH * 4, OP = OB + CH * 4;
  static constexpr int BUF = OP + CH * 4;              // one chunk's operands (a, b, positions)
  static constexpr int LDA = CH + 4;                   // fp32 64x64 A and T rows
  static constexpr int PA = 0, PT = PA + CH * LDA * 4, PPH = PT + CH * LDA * 4;
  static constexpr int PGAM = PPH + (int)kWsFrag, PRR = PGAM + CH * 4, PGS = PRR + CH * 4, PBS = PGS + CH * 4;
  static constexpr int PSS = PBS + CH * 4, PREP = PSS + CH * 4;
  static_assert(2 * BUF + PREP <= 160 * 1024, "LDS");
  static constexpr int BLK = 3 * TB / 1024 / NW;       // 1 KB loads of K, Q and V per wave
  static_assert(BLK * NW * 1024 == 3 * TB, "tiles divide over the waves");
  // FP8 inputs: a staging buffer holds one chunk's K, Q and V codes (row-major,
  // DK bytes per row) and, from X8, the per-row words a, b, positions, q
  // scales, v scales and k scales; the codes are decoded into one bf16 tile
  // buffer (TILES, the kq_off layout of the bf16 path) at the start of each
  // step
  static constexpr int TB8 = CH * DK, X8 = 3 * TB8, BUF8 = X8 + 6 * CH * 4, TILES = 3 * TB;
  static constexpr int XA = 0, XB = CH * 4, XP = 2 * CH * 4, XQS = 3 * CH * 4, XVS = 4 * CH * 4, XKS = 5 * CH * 4;
  static_assert(OB - OA == XB && OP - OA == XP, "per-row words at the same offsets in both layouts");
  static_assert(2 * BUF8 + TILES + PREP <= 160 * 1024, "LDS (FP8 inputs)");
  static constexpr int BLK8 = 3 * TB8 / 1024 / NW;     // 1 KB loads of codes per wave
  static_assert(BLK8 * NW * 1024 == 3 * TB8, "code tiles divide over the waves");
};

// F8: q, k, v arrive as E4M3 codes with fp32 scales per (token, head) row,
// q = rho q^, k = kappa k^, v = nu v^. Substituting these into the recurrence
// gives the same recurrence in the codes, S_t = a_t S_{t-1} (I - b'_t k^ k^T)
// + b'_t v'_t k^T with b' = b kappa^2 and v' = (nu / kappa) v^, and o_t =
// rho_t scale S_t q^_t: the kernel decodes the codes exactly into the bf16
// tiles (E4M3 values are bf16 values), replaces b by b' and scales V rows by
// nu / kappa where it forms R = V - gamma X in fp32, and scales each output
// row by rho; the state is the same state.
template <int DK, bool F8>
__global__ void __launch_bounds__(FusedCfg::NT, 1) gdn_fused_kernel(const int32_t* __restrict__ blob, GdnArgs args) {
  using F = FusedCfg;
  static_assert(DK == F::DK, "fused kernel is for dk = dv = 128");
  typedef unsigned short E;
  __shared__ __attribute__((aligned(16))) unsigned char buf0[F8 ? F::BUF8 : F::BUF];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[F8 ? F::BUF8 : F::BUF];
  __shared__ __attribute__((aligned(16))) unsigned char tiles8[F8 ? F::TILES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char prep[F::PREP];
  // a step's bf16 tiles and its per-row words
  auto tiles_of = [&](unsigned char* b) __attribute__((always_inline)) { return F8 ? tiles8 : b; };
  auto words_of = [&](unsigned char* b) __attribute__((always_inline)) { return b + (F8 ? F::X8 : F::OA); };

  if (!blob_ok(blob, args.guard)) return;
  const int level = args.level;
  const bool planned = args.lv_first >= 0;
  if (!planned && level > blob[MH_MAXDEPTH]) return;
  // without end states to store, leaf siblings run packed (GdnRec)
  const bool packed = args.seg_final == nullptr;
  const int32_t* __restrict__ level_off = blob + blob[packed ? MH_OFF_PACKOFF : MH_OFF_LEVELOFF];
  const int32_t* __restrict__ gdn_rec = blob + blob[packed ? MH_OFF_GDNPACK : MH_OFF_GDNREC];
  const int32_t* __restrict__ tok_pos = blob + blob[MH_OFF_TOKPOS];
  const int H = args.H;
  // the depth's first `take` segments are handled by gdn_coop_kernel
  const int take = planned ? args.lv_take : args.no_coop ? 0 : coop_segments(blob, level, H, DK);
  // (the packed list has its own offsets; its long segments lead each depth
  // in the level list's order, so `take` skips the same ones)
  const bool use_plan = planned && !packed;
  const int lv0 = (use_plan ? args.lv_first : level_off[level]) + take;
  const int nlev = (use_plan ? args.lv_first + args.lv_count : level_off[level + 1]) - lv0;
  const int nitems = nlev * H;
  // (the wave index as a scalar: branches on it stay scalar, so the compiler
  // keeps LDS accesses under them out of its waits for the LDS DMA below)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int e0 = 16 * w;  // this wave's state rows
  const E* __restrict__ Kg = (const E*)args.k;
  const E* __restrict__ Qg = (const E*)args.q;
  const E* __restrict__ Vg = (const E*)args.v;
  E* __restrict__ Og = (E*)args.o;
  const float* __restrict__ QSg = args.qs;
  const float* __restrict__ VSg = args.vs;
  const float* __restrict__ KSg = args.ks;
  // (the lambdas below use these copies, not args: a by-reference capture of
  // the kernel argument would put it in scratch memory)
  const float* __restrict__ Ag = args.a;
  const float* __restrict__ Bg = args.b;
  const float* __restrict__ root_state = args.root_state;
  float* __restrict__ seg_start_state = args.seg_start;
  float* __restrict__ seg_final_state = args.seg_final;
  const float oscale = args.scale;
  const size_t SZ = (size_t)DK * DK;

  float* As = (float*)(prep + F::PA);
  float* Ts = (float*)(prep + F::PT);
  float* gam = (float*)(prep + F::PGAM);
  float* rrv = (float*)(prep + F::PRR);
  float* gs = (float*)(prep + F::PGS);
  float* bs = (float*)(prep + F::PBS);
  int* ss = (int*)(prep + F::PSS);  // per row: first row of its segment in the chunk (0: at or before it)

  // a work item: segment (longest first within the depth) and head, from
  // the segment's record (one load)
  struct Item {
    int s, h, L, st, nck, src, fc, nsib;
  };
  auto item_at = [&](int it) __attribute__((always_inline)) {
    Item r;
    const int li = it / H;
    const int32_t* rec = gdn_rec + (size_t)(lv0 + li) * kGdnRecWords;
    const int4 a = *(const int4*)rec;
    const int4 b = *(const int4*)(rec + 4);
    r.s = __builtin_amdgcn_readfirstlane(a.x);
    r.st = __builtin_amdgcn_readfirstlane(a.y);
    r.L = __builtin_amdgcn_readfirstlane(a.z);
    r.src = __builtin_amdgcn_readfirstlane(a.w);
    r.fc = __builtin_amdgcn_readfirstlane(b.x);
    r.nsib = __builtin_amdgcn_readfirstlane(b.y);
    r.h = it - li * H;
    r.nck = (r.L + CH - 1) / CH;
    return r;
  };

  // loads of chunk ci of item r into buffer b: K, Q and V tiles in the kq_off
  // layout (chunk c of row i at c ^ kq_swz(i)), or with F8 their code tiles
  // row-major; rows past the chunk repeat its last row (they meet b = 0, so
  // they reach no output that is stored); the per-row words (a, b, positions,
  // and with F8 the q, v and k scales), one dword per lane, wave n loading the
  // n-th
  // The buffer's address goes through an empty asm statement: the compiler
  // then does not tie these LDS writes to the buffer, and adds no waits for
  // them before LDS accesses elsewhere in the step (it cannot tell the
  // buffers apart reliably); every read of a buffer follows the step's own
  // vmcnt(0) and barrier.
  auto issue = [&](unsigned char* b, const Item& r, int ci) __attribute__((always_inline)) {
    const int t0 = r.st + CH * ci, tl = t0 + min(CH, r.L - CH * ci) - 1;
    asm volatile("" : "+v"(b));
    if constexpr (F8) {
      // code tile i (K, Q, V): wave w loads its rows 8 w .. 8 w + 7 (1 KB);
      // lane l writes 16-byte position l % 8 of its row, which holds the
      // row's chunk code8_chunk(row, l % 8)
      static_assert(F::BLK8 == 3 && F::NW == 8 && F::TB8 == 8 * 1024, "one 1 KB block of each code tile per wave");
      const int row = 8 * w + (lane >> 3);
      const size_t g = ((size_t)min(t0 + row, tl) * H + r.h) * DK + 16 * code8_chunk(row, lane & 7);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const unsigned char* src = (const unsigned char*)(i == 0 ? Kg : (i == 1 ? Qg : Vg));
        __builtin_amdgcn_global_load_lds((const void*)(src + g), (lds_void_t*)(b + i * F::TB8 + w * 1024), 16, 0, 0);
      }
    } else {
      // 1 KB block n = 8 i + w: tile i / 2 (K, Q, V), block (i % 2) 8 + w of it
      static_assert(F::BLK == 6 && F::NW == 8 && F::TB == 16 * 1024, "two blocks of each tile per wave");
#pragma unroll
      for (int i = 0; i < F::BLK; ++i) {
        const int nb = (i % 2) * 8 + w;
        const int slot = nb * 64 + lane, row = slot / (DK / 8), pos = slot % (DK / 8);
        const E* src = i < 2 ? Kg : (i < 4 ? Qg : Vg);
        const size_t g = ((size_t)min(t0 + row, tl) * H + r.h) * DK + 8 * (pos ^ kq_swz(row, DK / 8));
        __builtin_amdgcn_global_load_lds((const void*)(src + g), (lds_void_t*)(b + (i / 2) * F::TB + nb * 1024), 16,
                                         0, 0);
      }
    }
    unsigned char* x = words_of(b);
    if (w < 2) {
      const float* src = w == 0 ? Ag : Bg;
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)min(t0 + lane, tl) * H + r.h),
                                       (lds_void_t*)(x + (w == 0 ? F::XA : F::XB)), 4, 0, 0);
    } else if (w == 2) {
      __builtin_amdgcn_global_load_lds((const void*)(tok_pos + min(t0 + lane, tl)), (lds_void_t*)(x + F::XP), 4,
                                       0, 0);
    } else if (F8 && w < 6) {
      const size_t ri = (size_t)min(t0 + lane, tl) * H + r.h;
      if (w == 3)
        __builtin_amdgcn_global_load_lds((const void*)(QSg + ri), (lds_void_t*)(x + F::XQS), 4, 0, 0);
      else if (w == 4)
        __builtin_amdgcn_global_load_lds((const void*)(VSg + ri), (lds_void_t*)(x + F::XVS), 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds((const void*)(KSg + ri), (lds_void_t*)(x + F::XKS), 4, 0, 0);
    }
  };

  // F8: decode the codes staged in b into the bf16 tiles (thread t: the 16
  // codes at 16-byte position t % 8 of row t / 8 of each tile), and replace
  // the row words b by b kappa^2 and the v scales by nu / kappa (wave 0)
  auto decode = [&](unsigned char* b) __attribute__((always_inline)) {
    const int row = tid >> 3, c0 = 16 * code8_chunk(row, tid & 7);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x4_t c = *(const u32x4_t*)(b + i * F::TB8 + row * DK + 16 * (tid & 7));
      unsigned pk[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // bytes 0, 1 and 2, 3 of dword d: codes c0 + 4 d + 0 .. 3 (exact in fp32 and in bf16)
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[d], false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[d], true);
        pk[2 * d] = pack_bf16x2(lo[0], lo[1]);
        pk[2 * d + 1] = pack_bf16x2(hi[0], hi[1]);
      }
      E* t = (E*)(tiles8 + i * F::TB);
      *(u32x4_t*)(t + kq_off<DK>(row, c0)) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      *(u32x4_t*)(t + kq_off<DK>(row, c0 + 8)) = u32x4_t{pk[4], pk[5], pk[6], pk[7]};
    }
    if (w == 0) {
      float* x = (float*)(b + F::X8);
      const float kap = x[F::XKS / 4 + lane];
      x[F::XB / 4 + lane] *= kap * kap;
      x[F::XVS / 4 + lane] /= kap;
    }
  };

  // The state (St: lane (c16, q4) holds S[e0 + c16][16 db + 4 q4 + r], S^T
  // blocks) and its products with the chunk, X = K S^T and Y^T = S Q^T
  // (block I: rows 16 I + 4 q4 + r of X and Y, state row e0 + c16), which
  // need nothing from the chunk preparation.
  f32x4_t St[DK / 16], X[4], Yt[4];
  auto state_products = [&](const unsigned char* t) __attribute__((always_inline)) {
    const E* Ks = (const E*)t;
    const E* Qs = (const E*)(t + F::OQ);
#pragma unroll
    for (int I = 0; I < 4; ++I) X[I] = Yt[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < DK / 32; ++f) {
      bf16x8_t sh, sl;
      reg_frag<true>(St, f, sh, sl);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const bf16x8_t ka = kq_frag<DK>(Ks, 16 * I + c16, f, q4);
        const bf16x8_t qb = kq_frag<DK>(Qs, 16 * I + c16, f, q4);
        X[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, sh, X[I], 0, 0, 0);
        X[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, sl, X[I], 0, 0, 0);
        Yt[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sh, qb, Yt[I], 0, 0, 0);
        Yt[I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl, qb, Yt[I], 0, 0, 0);
      }
    }
  };

  // ---- chunk preparation (operands of the chunk in b). Waves 0-3 form row
  // block w of P = QK^T * Gamma (as hi / lo fragments), waves 4-7 row block
  // w - 4 of A and the inverse of its diagonal block; wave 0 then computes
  // the decays, which the products do not need. Each wave then forms its
  // state products (they overlap the diagonal inverses on the same SIMDs).
  // (t: the bf16 tiles; x: the per-row words; c8: with F8, the code tiles)
  auto prep_chunk = [&](const unsigned char* t, const unsigned char* x, const unsigned char* c8, int len)
                        __attribute__((always_inline)) {
    const E* Ks = (const E*)t;
    const E* Qs = (const E*)(t + F::OQ);
    const int rb = w & 3;      // this wave's row block
    const bool kk = w >= 4;    // K K^T (A) rather than Q K^T (P)
    // Xt_J = K_J X_rb^T for J <= rb, X = Q or K (16x16x32 bf16, k-order of a
    // 16-byte row read); lane (c16, q4) holds row i = 16 rb + c16 of XK^T at
    // columns j = 16 J + 4 q4 + r
    f32x4_t xt[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) xt[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
      // the products of the codes on the FP8 matrix cores (E4M3 x E4M3, unit
      // block scales, one 16x16x128 product per block): lane (c16, q4) holds
      // the 32 codes at k = 32 q4 .. 32 q4 + 31 of its row in both operands
      const unsigned char* X8 = c8 + (kk ? 0 : F::TB8);
      // the 32 codes of row r at k = 32 q4 .. 32 q4 + 31: chunks 2 q4 and 2 q4 + 1
      auto codes32 = [&](const unsigned char* t, int r) __attribute__((always_inline)) {
        const u32x4_t lo = *(const u32x4_t*)(t + r * DK + 16 * code8_chunk(r, 2 * q4));
        const u32x4_t hi = *(const u32x4_t*)(t + r * DK + 16 * code8_chunk(r, 2 * q4 + 1));
        return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      const i32x8_t bx = codes32(X8, 16 * rb + c16);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= rb) {
          const i32x8_t aK = codes32(c8, 16 * J + c16);
          xt[J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aK, bx, xt[J], 0, 0, 0, 127, 0, 127);
        }
      }
    } else {
      const E* Xs = kk ? Ks : Qs;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const bf16x8_t bx = *(const bf16x8_t*)(Xs + kq_off<DK>(16 * rb + c16, 32 * ks + 8 * q4));
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          if (J <= rb) {
            const bf16x8_t aK = *(const bf16x8_t*)(Ks + kq_off<DK>(16 * J + c16, 32 * ks + 8 * q4));
            xt[J] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aK, bx, xt[J], 0, 0, 0);
          }
        }
      }
    }
    if (w == 0) {
      // g restarts at each segment's first row (packed siblings): from the
      // row's position in its segment, sr = the row its segment starts at
      // (rows past the chunk hold the last row's position and take its sr,
      // so they keep its decay: g of the last row is the chunk's total)
      const float a = ((const float*)(x + F::XA))[lane];
      const float L = wave_incl_scan(lane < len ? log_gate(a) : 0.f, lane);
      const int sr = min(lane, len - 1) - ((const int*)(x + F::XP))[lane];
      const float Lb = __shfl(L, sr > 0 ? sr - 1 : 0);
      const float la = sr > 0 ? L - Lb : L;
      const float gl = lane_val(la, CH - 1);
      ss[lane] = sr > 0 ? sr : 0;
      gs[lane] = la;
      bs[lane] = lane < len ? ((const float*)(x + F::XB))[lane] : 0.f;
      gam[lane] = __expf(la);
      rrv[lane] = __expf(gl - la);
    }
    lds_barrier();  // g, b, gamma
    const int i = 16 * rb + c16;
    const float gi = gs[i], bi = bs[i];
    const int si = ss[i];
    f32x4_t gj[4];
    int4 sj[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      gj[J] = *(const f32x4_t*)(gs + 16 * J + 4 * q4);
      sj[J] = *(const int4*)(ss + 16 * J + 4 * q4);
    }
    // (i, j) in one segment: same first row
    auto same = [&](int J, int r) __attribute__((always_inline)) {
      return (r == 0 ? sj[J].x : r == 1 ? sj[J].y : r == 2 ? sj[J].z : sj[J].w) == si;
    };
    if (!kk) {
      // P = Q K^T * Gamma (j <= i), stored as fragments
      f32x4_t pv[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * J + 4 * q4 + r;
          pv[J][r] = J <= rb && j <= i && same(J, r) ? __expf(gi - gj[J][r]) * xt[J][r] : 0.f;
        }
      }
      u32x4_t* Pw = (u32x4_t*)(prep + F::PPH);
#pragma unroll
      for (int kf = 0; kf < 2; ++kf) {
        if (kf < frag_nk(rb)) {
          const int fb = frag_tri(rb) + kf;
          u32x2_t h0, l0, h1, l1;
          split4(pv[2 * kf], h0, l0);
          split4(pv[2 * kf + 1], h1, l1);
          Pw[(2 * fb) * 64 + lane] = u32x4_t{h0.x, h0.y, h1.x, h1.y};
          Pw[(2 * fb + 1) * 64 + lane] = u32x4_t{l0.x, l0.y, l1.x, l1.y};
        }
      }
    } else {
      // A = strictly_lower(diag(b) K K^T * Gamma)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= rb) {
          f32x4_t av;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * J + 4 * q4 + r;
            av[r] = j < i && same(J, r) ? bi * __expf(gi - gj[J][r]) * xt[J][r] : 0.f;
          }
          *(f32x4_t*)(As + i * F::LDA + 16 * J + 4 * q4) = av;
        }
      }
      // the inverse of diagonal block rb of I + A (its rows of A are this
      // wave's own stores)
      diag_inverse(As, Ts, F::LDA, 16 * rb, lane);
    }
    state_products(t);
    lds_barrier();  // P, A, the diagonal inverses and the decays are complete
  };

  // ---- one chunk of the scan for this wave's slice (operands in b; P, A,
  // the diagonal inverses and the decays in prep; X and Y^T formed)
  auto scan_chunk = [&](const unsigned char* t, const unsigned char* x, const Item& r, int t0, int len,
                        bool need_state) __attribute__((always_inline)) {
    const E* Ks = (const E*)t;
    const E* Vs = (const E*)(t + F::OV);
    const u32x4_t* Ph = (const u32x4_t*)(prep + F::PPH);
    // (2) R = V - gamma X: lane (c16, q4), block I holds R[16 I + 4 q4 + r][e0 + c16]
    f32x4_t R[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const s16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(Vs + kq_off<DK>(16 * I + 4 * q4 + (c16 >> 2), e0 + 4 * (c16 & 3))));
      const f32x4_t g4 = *(const f32x4_t*)(gam + 16 * I + 4 * q4);
      // (F8: V rows times nu / kappa)
      const f32x4_t f4 = F8 ? *(const f32x4_t*)(x + F::XVS + 4 * (16 * I + 4 * q4)) : f32x4_t{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) R[I][k] = fmaf(-g4[k], X[I][k], bf16_val((unsigned short)v4[k]) * f4[k]);
    }
    // (3) U = T'' R = (I + A)^-1 diag(b) R by block forward substitution:
    // U_I = T_II (b_I R_I - sum_{K<I} A_IK U_K), T_II the inverse of the
    // diagonal block of I + A (16x16x16 bf16 hi / lo products: a block's
    // accumulator layout is the B operand layout of the next product)
    f32x4_t U[4];
    s16x4_t ubh[3], ubl[3];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4_t acc = R[I] * *(const f32x4_t*)(bs + 16 * I + 4 * q4);
#pragma unroll
      for (int K = 0; K < I; ++K) {
        const f32x4_t a4 = -*(const f32x4_t*)(As + (16 * I + c16) * F::LDA + 16 * K + 4 * q4);
        u32x2_t ah, al;
        split4(a4, ah, al);
        const s16x4_t ahs = __builtin_bit_cast(s16x4_t, ah), als = __builtin_bit_cast(s16x4_t, al);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahs, ubh[K], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahs, ubl[K], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(als, ubh[K], acc, 0, 0, 0);
      }
      u32x2_t ch, cl, th, tl;
      split4(acc, ch, cl);
      split4(*(const f32x4_t*)(Ts + (16 * I + c16) * F::LDA + 16 * I + 4 * q4), th, tl);
      const s16x4_t ths = __builtin_bit_cast(s16x4_t, th), tls = __builtin_bit_cast(s16x4_t, tl);
      const s16x4_t chs = __builtin_bit_cast(s16x4_t, ch), cls = __builtin_bit_cast(s16x4_t, cl);
      f32x4_t u = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ths, chs, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      u = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ths, cls, u, 0, 0, 0);
      u = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tls, chs, u, 0, 0, 0);
      U[I] = u;
      if (I < 3) {
        u32x2_t uh, ul;
        split4(u, uh, ul);
        ubh[I] = __builtin_bit_cast(s16x4_t, uh);
        ubl[I] = __builtin_bit_cast(s16x4_t, ul);
      }
    }
    // (4) O^T = scale (gamma Y^T + U^T P^T): lane (c16, q4), block I holds
    // O[16 I + c16][e0 + 4 q4 + r]; stored at once
    bf16x8_t uh[2], ul[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) reg_frag<true>(U, f, uh[f], ul[f]);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4_t Zt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kf = 0; kf < frag_nk(I); ++kf) {
        const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, Ph[(frag_tri(I) + kf) * 128 + lane]);
        const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, Ph[(frag_tri(I) + kf) * 128 + 64 + lane]);
        Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[kf], ph, Zt, 0, 0, 0);
        Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul[kf], ph, Zt, 0, 0, 0);
        Zt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[kf], pl, Zt, 0, 0, 0);
      }
      const int i = 16 * I + c16;
      // (F8: the row's q scale rho)
      const float osc = F8 ? oscale * ((const float*)(x + F::XQS))[i] : oscale;
      const f32x4_t o = osc * (gam[i] * Yt[I] + Zt);
      if (i < len) {
        E* d = Og + ((size_t)(t0 + i) * H + r.h) * DK + e0 + 4 * q4;
        *(u32x2_t*)d = u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    }
    if (!need_state) return;
    // (5) S^T = gamma_C S^T + K^T U',  U' = diag(gamma_C / gamma) U
#pragma unroll
    for (int I = 0; I < 4; ++I) U[I] *= *(const f32x4_t*)(rrv + 16 * I + 4 * q4);
#pragma unroll
    for (int f = 0; f < 2; ++f) reg_frag<true>(U, f, uh[f], ul[f]);
    const float gC = gam[CH - 1];
#pragma unroll
    for (int db = 0; db < DK / 16; ++db) St[db] *= gC;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int db = 0; db < DK / 16; ++db) {
        const bf16x8_t kt = kt_frag<DK>(Ks, 16 * db, f, lane);
        St[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, uh[f], St[db], 0, 0, 0);
        St[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, ul[f], St[db], 0, 0, 0);
      }
  };

  // ---- the workgroup's items, chunk by chunk; loads run one chunk ahead
  // through two buffers (the loop is unrolled by two so each step reads and
  // fills fixed buffers).
  // Items are handed out longest first: a workgroup's first item is static
  // (blockIdx.x), later ones come from the blob's counter (value c: item
  // c + gridDim.x), so a workgroup that ends a long segment early takes the
  // next one (greedy longest-processing-time order over the depth's very
  // uneven segments). The next item is requested just in time: at the start
  // of the step that loads the current item's last chunk (thread 0's atomic),
  // published after that step's preparation (the item in s_res, its record
  // copied into s_rec by wave 0's DMA) and taken at the next step's start,
  // after its vmcnt(0) and barrier, so no wave waits for a global load there.
  // The last workgroup to finish resets the counters. A launch with no more
  // items than workgroups makes no request (every item is a first item).
  __shared__ int s_res;
  __shared__ __attribute__((aligned(16))) int32_t s_rec[kGdnRecWords];
  int32_t* __restrict__ ctr = args.ctr;
  int tk = 0;  // thread 0: the requested item
  const bool dyn = nitems > (int)gridDim.x;
  auto request = [&]() __attribute__((always_inline)) {
    if (tid == 0) tk = dyn ? atomicAdd(ctr, 1) + (int)gridDim.x : nitems;
  };
  auto publish = [&]() __attribute__((always_inline)) {
    if (w == 0) {
      const int r = __builtin_amdgcn_readfirstlane(tk);
      if (lane == 0) s_res = r;
      if (r < nitems && lane < kGdnRecWords) {
        unsigned char* d = (unsigned char*)s_rec;
        asm volatile("" : "+v"(d));  // (as in issue: no compiler waits for this DMA)
        __builtin_amdgcn_global_load_lds((const void*)(gdn_rec + (size_t)(lv0 + r / H) * kGdnRecWords + lane),
                                         (lds_void_t*)d, 4, 0, 0);
      }
    }
  };
  int it = blockIdx.x;
  if (it < nitems) {
    Item cur = item_at(it);
    int ci = 0;
    issue(buf0, cur, 0);
    if (cur.nck == 1) {  // the next chunk is the next item's
      request();
      publish();
    }
    const size_t srow = (size_t)(e0 + c16) * DK + 4 * q4;
    auto step = [&](unsigned char* b, unsigned char* other) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of the chunk landed
      lds_barrier();                       // B0: every wave's loads landed; `other` is free
      // the chunk after (cur, ci): cur's next, or the published item's first
      Item nx = cur;
      int nci = ci + 1;
      bool has_next = true;
      if (nci >= cur.nck) {
        const int r = __builtin_amdgcn_readfirstlane(s_res);
        has_next = r < nitems;
        if (has_next) {
          const int li = r / H;
          nx.s = __builtin_amdgcn_readfirstlane(s_rec[0]);
          nx.st = __builtin_amdgcn_readfirstlane(s_rec[1]);
          nx.L = __builtin_amdgcn_readfirstlane(s_rec[2]);
          nx.src = __builtin_amdgcn_readfirstlane(s_rec[3]);
          nx.fc = __builtin_amdgcn_readfirstlane(s_rec[4]);
          nx.nsib = __builtin_amdgcn_readfirstlane(s_rec[5]);
          nx.h = r - li * H;
          nx.nck = (nx.L + CH - 1) / CH;
        }
        nci = 0;
      }
      // request the item after nx when nx's chunk is its last
      const bool req = has_next && nci + 1 >= nx.nck;
      if (req) request();
      // start state at an item's first chunk, loaded here (before the next
      // chunk's loads) so that its latency hides behind the chunk
      // preparation; copied into the start slot of each of the item's
      // segments except the one the parent's item wrote it to (the first
      // child)
      if (ci == 0) {
        const float* src = nullptr;
        if (cur.src < 0) {
          if (root_state) src = root_state + ((size_t)(-1 - cur.src) * H + cur.h) * SZ;
        } else {
          src = seg_start_state + ((size_t)cur.src * H + cur.h) * SZ;
        }
#pragma unroll
        for (int db = 0; db < DK / 16; ++db)
          St[db] = src ? *(const f32x4_t*)(src + srow + 16 * db) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      if (has_next) issue(other, nx, nci);
      const int t0 = cur.st + CH * ci, len = min(CH, cur.L - CH * ci);
      if constexpr (F8) {
        decode(b);
        lds_barrier();  // the decoded tiles and the scaled row words
      }
      prep_chunk(tiles_of(b), words_of(b), b, len);
      if (req) publish();
      if (ci == 0) {
        for (int q = 0; q < cur.nsib; ++q) {
          const int sq = cur.s + q;
          if (sq == cur.src) continue;
          float* own = seg_start_state + ((size_t)sq * H + cur.h) * SZ;
#pragma unroll
          for (int db = 0; db < DK / 16; ++db) *(f32x4_t*)(own + srow + 16 * db) = St[db];
        }
      }
      const bool last = ci + 1 == cur.nck;
      const int fc = cur.fc;
      const bool need_state = !last || fc >= 0 || seg_final_state != nullptr;
      scan_chunk(tiles_of(b), words_of(b), cur, t0, len, need_state);
      if (last) {
        if (seg_final_state) {
          float* d = seg_final_state + ((size_t)cur.s * H + cur.h) * SZ;
#pragma unroll
          for (int db = 0; db < DK / 16; ++db) *(f32x4_t*)(d + srow + 16 * db) = St[db];
        }
        if (fc >= 0) {
          float* d = seg_start_state + ((size_t)fc * H + cur.h) * SZ;
#pragma unroll
          for (int db = 0; db < DK / 16; ++db) *(f32x4_t*)(d + srow + 16 * db) = St[db];
        }
      }
      // the prep region is rewritten by the next chunk only after its B0 and
      // decay barrier, which every wave reaches after this scan
      cur = nx;
      ci = nci;
      return has_next;
    };
    for (;;) {
      if (!step(buf0, buf1)) break;
      if (!step(buf1, buf0)) break;
    }
  }
  if (tid == 0) {
    __threadfence();  // (the last request has returned)
    if (atomicAdd(ctr + 1, 1) == (int)gridDim.x - 1) {
      // every other workgroup has made its last request: reset for the next launch
      atomicExch(ctr, 0);
      atomicExch(ctr + 1, 0);
    }
  }
}

template <bool BF16, int DK>
fork_status launch_gdn_t(const fork_meta* m, GdnArgs a, hipStream_t stream) {
  const bool cap = stream_capturing(stream);
  const int cus = device_cu_count();
  const int sgrid = (cus + 7) / 8 * 8;  // one workgroup per CU (LDS); a multiple of 8: item i runs on XCD i mod 8
  // bf16 with dk = 128: the fused kernel prepares and scans every segment
  // except the latency-bound long ones gdn_coop_kernel takes, whose chunks
  // alone go through gdn_prep_kernel and the workspace
  constexpr bool FUSED = BF16 && DK == FusedCfg::DK;
  a.sgrid = sgrid;
  a.prep_coop_only = FUSED ? 1 : 0;
  // per depth: [first segment in the level list, segments, coop's share]
  // when the host plans (outside capture)
  const int levels = cap ? m->caps.depth_cap + 1 : m->max_depth + 1;
  bool any_coop = false;
  if (!cap) {
    for (int lv = 0; lv < levels && lv < FORK_PLAN_DEPTHS; ++lv) {
      const long long coop_items = (long long)m->level_long[lv] * ((a.H + 7) / 8) * 8 * (DK / 16);
      any_coop |= BF16 && m->level_long[lv] > 0 && coop_items <= sgrid;
    }
    if (m->max_depth >= FORK_PLAN_DEPTHS) any_coop = true;  // (unplanned depths decide in the kernels)
  }
  if (!FUSED || cap || any_coop) {
    int grid = PrepCfg<BF16, DK>::PER_CU * cus;
    if (!cap && !FUSED) {
      const long long items = (long long)m->num_chunks * a.H;
      if (items < grid) grid = (int)(items > 0 ? items : 1);
    }
    hipLaunchKernelGGL((gdn_prep_kernel<BF16, DK>), dim3(grid), dim3(256), 0, stream, a.blob, a);
    FORK_HIP_CHECK(hipGetLastError());
  }
  // Scan launches per depth (children start after their parents ended): the
  // chunk-cooperative kernel for a latency-bound set of long segments, the
  // fused (bf16, dk 128) or per-slice kernel for the rest. Under capture,
  // every depth up to the capacity is recorded with both kernels, which split
  // the depth from the blob; depths beyond the current tree exit at once.
  int first = 0;  // first segment of the depth in the blob's level list
  for (int lv = 0; lv < levels; ++lv) {
    a.level = lv;
    bool run_coop = BF16, run_scan = true;
    a.lv_first = a.lv_count = a.lv_take = -1;
    if (!cap && lv < FORK_PLAN_DEPTHS) {
      // the kernels' split of the depth (coop_segments), decided here so that
      // launches without work are skipped
      const int nseg = m->level_segs[lv], nlong = m->level_long[lv];
      const long long coop_items = (long long)nlong * ((a.H + 7) / 8) * 8 * (DK / 16);
      const int take = BF16 && coop_items <= sgrid ? nlong : 0;
      a.lv_first = first;
      a.lv_count = nseg;
      a.lv_take = take;
      run_coop = take > 0;
      run_scan = nseg - take > 0;
      first += nseg;
    }
    if constexpr (BF16) {
      if (run_coop) {
        hipLaunchKernelGGL((gdn_coop_kernel<DK>), dim3(sgrid), dim3(CoopCfg<DK>::NT), 0, stream, a.blob, a);
        FORK_HIP_CHECK(hipGetLastError());
      }
    }
    if (run_scan) {
      if constexpr (FUSED) {
        int grid = sgrid;
        if (!cap && a.lv_first >= 0) {
          const long long items = (long long)(a.lv_count - a.lv_take) * a.H;
          if (items < grid) grid = (int)items;
        }
        hipLaunchKernelGGL((gdn_fused_kernel<DK, false>), dim3(grid), dim3(FusedCfg::NT), 0, stream, a.blob, a);
      } else {
        hipLaunchKernelGGL((gdn_scan_kernel<BF16, DK>), dim3(sgrid), dim3(ScanCfg<BF16, DK>::NT), 0, stream,
                           a.blob, a);
      }
      FORK_HIP_CHECK(hipGetLastError());
    }
  }
  return FORK_OK;
}

// FP8 inputs: every depth runs on gdn_fused_kernel<128, true> (no
// chunk-cooperative path, hence no preparation kernel and no workspace). Under
// capture every depth up to the capacity is recorded; depths beyond the
// current tree exit at once.
fork_status launch_gdn_fp8_t(const fork_meta* m, GdnArgs a, hipStream_t stream) {
  const bool cap = stream_capturing(stream);
  const int sgrid = (device_cu_count() + 7) / 8 * 8;
  a.sgrid = sgrid;
  a.no_coop = 1;
  const int levels = cap ? m->caps.depth_cap + 1 : m->max_depth + 1;
  int first = 0;
  for (int lv = 0; lv < levels; ++lv) {
    a.level = lv;
    a.lv_first = a.lv_count = a.lv_take = -1;
    int grid = sgrid;
    if (!cap && lv < FORK_PLAN_DEPTHS) {
      const int nseg = m->level_segs[lv];
      a.lv_first = first;
      a.lv_count = nseg;
      a.lv_take = 0;
      first += nseg;
      if (nseg == 0) continue;
      const long long items = (long long)nseg * a.H;
      if (items < grid) grid = (int)items;
    }
    hipLaunchKernelGGL((gdn_fused_kernel<128, true>), dim3(grid), dim3(FusedCfg::NT), 0, stream, a.blob, a);
    FORK_HIP_CHECK(hipGetLastError());
  }
  return FORK_OK;
}

}  // namespace

fork_status launch_gdn_fp8(const fork_meta* m, const void* q8, const float* qs, const void* k8, const float* ks,
                           const void* v8, const float* vs, const float* a, const float* b, const float* root_state,
                           void* o, float* seg_start_state, float* seg_final_state, int H, float scale,
                           hipStream_t stream) {
  GdnArgs g;
  g.blob = (const int32_t*)m->dev;
  g.q = q8;
  g.k = k8;
  g.v = v8;
  g.qs = qs;
  g.ks = ks;
  g.vs = vs;
  g.a = a;
  g.b = b;
  g.root_state = root_state;
  g.o = o;
  g.seg_start = seg_start_state;
  g.seg_final = seg_final_state;
  g.ws = nullptr;
  g.ctr = (int32_t*)m->dev + kGdnCtrWord;
  g.guard = blob_guard(m->caps);
  g.H = H;
  g.scale = scale;
  g.level = 0;
  g.lv_first = g.lv_count = g.lv_take = -1;
  g.prep_coop_only = 0;
  g.sgrid = 0;
  g.no_coop = 1;
  return launch_gdn_fp8_t(m, g, stream);
}

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
  g.ctr = (int32_t*)m->dev + kGdnCtrWord;
  g.guard = blob_guard(m->caps);
  g.H = H;
  g.scale = scale;
  g.level = 0;
  g.lv_first = g.lv_count = g.lv_take = -1;
  g.prep_coop_only = 0;
  g.sgrid = 0;
  g.qs = g.ks = g.vs = nullptr;
  g.no_coop = 0;
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
