// Tree-masked flash attention over the flattened decision stream (gfx950).
//
// Semantics (Flide, kongchang.com page, sections "attention masks and
// probability distortion" and "ForkAttention: exact forking in GPU indices"):
// token t of segment s attends to every token of s's ancestor segments and to
// the tokens of s up to t; siblings never see each other, so each branch gets
// exactly the softmax of an isolated forward pass.
//
// Work decomposition. A work item is (query tile, kv head). A query tile holds
// up to 256 rows = tokens x GQA heads of one kv head, taken from one segment or
// from several consecutive short sibling segments (which share all ancestor
// keys). The item walks the ancestor segments' key ranges (fully visible, no
// mask except the ragged end of a range) and then its own range (masked by
// seg_start(row) <= j <= t(row)). Every 64-key K/V tile is staged in LDS once
// and used by all 256 rows, so a long shared prefix is read once per tile of
// packed branch queries instead of once per branch.
//
// Kernel shape: 512 threads = 8 wave64s (two per SIMD, one workgroup per CU),
// each wave owns 32 of the tile's 256 query rows, so every staged key/value
// tile feeds 256 rows.
// S^T = K Q^T and O^T = V^T P^T on MFMA (32x32x16 bf16, or 32x32x2 f32): with
// keys on the MFMA M dimension, each lane holds one query row's scores in its
// registers, so the online-softmax row max needs one cross-lane step and the
// row sum none until the end. bf16 tiles arrive in LDS by DMA, row-major, and
// the V^T operand of O^T = V^T P^T comes from transposing LDS reads; fp32
// tiles are staged through registers, V transposed on its way to LDS.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace fork {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kAttnThreads = 512;  // 8 waves per workgroup, one workgroup per CU

// F8: queries and keys are E4M3 codes with one fp32 scale per (token, head)
// row, and S = K Q^T runs on the FP8 matrix cores (32x32x64); values stay
// bf16. Only with bf16 values and D = 128.
template <bool BF16, int D, bool F8 = false>
struct AttnCfg {
  static_assert(!F8 || (BF16 && D == 128), "FP8 scores with bf16 values, head_dim 128");
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int EPC = 16 / ESZ;                 // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per K/V row
  // fp32 tiles: K row stride in LDS; V transposed [d][key] and its pitch
  static constexpr int KS = D + EPC;
  static constexpr int VS = kAttnKeys + 4;
  static constexpr int VROWS = D;                      // rows of the fp32 V^T tile
  static constexpr int NKF = BF16 ? D / 16 : D / 2;    // MFMA k-steps over D
  static constexpr int NDB = D / 32;                   // 32-row d blocks of O^T
  // bf16 tiles: unpadded rows of D elements (CPR 16-byte chunks), one K and
  // one V tile per buffer
  static constexpr int TILE_BYTES = kAttnKeys * D * ESZ;
  // a buffer: the K tile (E4M3 rows of D bytes with F8), the V tile (bf16) at
  // V_OFF, and with F8 the tile's 64 key scales at KS_OFF; at least 32 KB
  // (four waves' output rows are staged through a buffer)
  static constexpr int V_OFF = F8 ? kAttnKeys * D : TILE_BYTES;
  static constexpr int KS_OFF = V_OFF + TILE_BYTES;
  static constexpr int F8_BYTES = KS_OFF + kAttnKeys * 4 > 32 * 1024 ? KS_OFF + kAttnKeys * 4 : 32 * 1024;
  static constexpr int BUF_BYTES = F8 ? F8_BYTES
                                 : BF16 ? 2 * TILE_BYTES
                                        : (kAttnKeys * KS > VROWS * VS ? kAttnKeys * KS : VROWS * VS) * ESZ;
};

// K/V tiles are written by DMA as whole 16-byte chunks, unpadded, with the
// chunks of each row permuted so that the reads below meet no LDS bank
// conflicts on the 64 banks of 4 bytes (a 16-byte read serves 16 lanes per
// cycle, an 8-byte read 32). CPR: chunks per row. K: chunk c of key row r at
// c ^ (r mod CPR), so the 16 rows one cycle reads at one chunk (CPR = 16) take
// 16 different bank groups. V: at c ^ 4 (r mod 4) (CPR = 16), so the
// transposing reads of 4 rows x 2 adjacent chunk pairs that one cycle serves
// take 8 different 32-byte bank groups; c ^ 2 (r mod 4) for rows of 8 chunks.
template <int CPR>
__device__ __forceinline__ int k_chunk_pos(int r, int c) {
  return c ^ (r & (CPR - 1));
}
// E4M3 key rows are 128 bytes (8 chunks), two rows per 256-byte bank cycle:
// chunk c of row r at c ^ ((r / 2) mod 8), so 16 consecutive rows read at one
// chunk take 16 different bank groups.
__device__ __forceinline__ int k8_chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }

// Lanes l and l ^ 32 hold one query row's scores. lane_pair gives every lane
// both of their values (its own and its partner's, in either order) by one
// lane swap between the wave's halves, with no round trip through LDS: lanes
// below 32 get (own, lane l + 32's), the others (lane l - 32's, own).
struct LanePair {
  float a, b;
};
__device__ __forceinline__ LanePair lane_pair(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
template <int CPR>
__device__ __forceinline__ int v_chunk_pos(int r, int c) {
  return CPR >= 16 ? c ^ ((r & 3) << 2) : c ^ ((r & 3) << 1);
}

// DMA of keys [j0, j0 + 64) of kv head g (rows past jmax repeat row jmax) into
// one K/V buffer: the buffer is a sequence of 1 KB blocks, block n filled by
// one 64-lane instruction (lane l writes 16 bytes at n * 1024 + 16 l); each
// wave issues its share of the blocks.
typedef __attribute__((address_space(3))) void lds_void_t;
// FP8 keys: the K tile is 64 rows of D bytes, chunk c of row r at
// k8_chunk_pos(r, c); each wave also loads 8 of the tile's key scales (one dword per
// lane, lanes 0-7) to KS_OFF, so every wave issues the same number of DMAs.
template <int D>
__device__ __forceinline__ void kv_dma_f8(unsigned char* buf, const unsigned char* __restrict__ K8,
                                          const float* __restrict__ kscale, const unsigned short* __restrict__ V,
                                          int j0, int jmax, int g, int Hkv, int wave, int lane) {
  using C = AttnCfg<true, D, true>;
  constexpr int KCPR = D / 16;                        // 16-byte chunks per fp8 row
  constexpr int VCPR = D / 8;                         // 16-byte chunks per bf16 row
  constexpr int NW = kAttnThreads / 64;
  static_assert(kAttnKeys * D / 1024 == NW && kAttnKeys * D * 2 / 1024 == 2 * NW, "one K and two V blocks per wave");
  {
    const int slot = wave * 64 + lane, r = slot / KCPR, pos = slot % KCPR;
    const size_t row = (size_t)min(j0 + r, jmax) * Hkv + g;
    __builtin_amdgcn_global_load_lds((const void*)(K8 + row * D + 16 * k8_chunk_pos(r, pos)),
                                     (lds_void_t*)(buf + wave * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = wave * 2 + i;
    const int slot = n * 64 + lane, r = slot / VCPR, pos = slot % VCPR;
    const size_t row = (size_t)min(j0 + r, jmax) * Hkv + g;
    __builtin_amdgcn_global_load_lds((const void*)(V + row * D + 8 * v_chunk_pos<VCPR>(r, pos)),
                                     (lds_void_t*)(buf + C::V_OFF + n * 1024), 16, 0, 0);
  }
  if (lane < 8) {
    const int r = 8 * wave + lane;
    __builtin_amdgcn_global_load_lds((const void*)(kscale + (size_t)min(j0 + r, jmax) * Hkv + g),
                                     (lds_void_t*)(buf + C::KS_OFF + 32 * wave), 4, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void kv_dma(unsigned char* buf, const unsigned short* __restrict__ K,
                                       const unsigned short* __restrict__ V, int j0, int jmax, int g, int Hkv,
                                       int wave, int lane) {
  constexpr int CPR = D / 8;                          // 16-byte chunks per row
  constexpr int NBLK = kAttnKeys * D * 2 / 1024;      // 1 KB blocks per tile
  constexpr int PER_WAVE = NBLK / (kAttnThreads / 64);
  static_assert(PER_WAVE * (kAttnThreads / 64) == NBLK, "tile blocks must divide over the waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int n = wave * PER_WAVE + i;
    const int slot = n * 64 + lane, r = slot / CPR, pos = slot % CPR;
    const size_t row = (size_t)min(j0 + r, jmax) * Hkv + g;
    __builtin_amdgcn_global_load_lds((const void*)(K + row * D + 8 * k_chunk_pos<CPR>(r, pos)),
                                     (lds_void_t*)(buf + n * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(V + row * D + 8 * v_chunk_pos<CPR>(r, pos)),
                                     (lds_void_t*)(buf + kAttnKeys * D * 2 + n * 1024), 16, 0, 0);
  }
}

struct AttnArgs {
  const int32_t* blob;
  const void* q;
  const void* k;
  const void* v;
  const void* kc;  // key/value cache of resumed contexts (null: none)
  const void* vc;
  void* o;
  float* lse;
  const float* qs;    // FP8 scores: scales of the q rows [T, H] and the k rows [T, Hkv]
  const float* ks;
  unsigned char* ws;  // partial results of split tiles: [slot][kv head] x (rows x D outputs, rows lse)
  int32_t* ctr;  // the blob's work counters: next item per XCD (8), finished workgroups
  BlobGuard guard;
  int H, Hkv, G;
  float scale_log2;  // softmax scale * log2(e)
};

// fp32 key/value tile of 64 keys held in registers between its global load and
// its LDS store, so the next tile's loads are in flight while the current
// tile is being computed (bf16 tiles go to LDS by DMA instead).
template <bool BF16, int D>
struct KVRegs {
  static_assert(!BF16, "bf16 tiles are staged by DMA");
  using C = AttnCfg<BF16, D>;
  static constexpr int KT = kAttnKeys * C::CPR / kAttnThreads;  // 16-byte K loads per thread
  // fp32 V is transposed on its way to LDS, in tasks of 4 keys x 16 bytes
  static constexpr int VTASKS = (kAttnKeys / 4) * C::CPR;
  static constexpr int VT = (VTASKS + kAttnThreads - 1) / kAttnThreads;
  static_assert(KT * kAttnThreads == kAttnKeys * C::CPR, "K tile loads must divide evenly");
  u32x4_t k[KT];
  u32x4_t v[VT][4];
};

// Global loads of keys [j0, j0 + 64) of kv head g; rows past `jmax` repeat
// row jmax (in range; their scores are masked).
template <bool BF16, int D, typename E>
__device__ __forceinline__ void kv_load(KVRegs<BF16, D>& r, const E* __restrict__ K,
                                        const E* __restrict__ V, int j0, int jmax, int g, int Hkv,
                                        int tid) {
  using C = AttnCfg<BF16, D>;
  using R = KVRegs<BF16, D>;
#pragma unroll
  for (int i = 0; i < R::KT; ++i) {
    const int task = tid + kAttnThreads * i;
    const int row = task / C::CPR, ch = task % C::CPR;
    const int j = min(j0 + row, jmax);
    r.k[i] = *(const u32x4_t*)(K + ((size_t)j * Hkv + g) * D + ch * C::EPC);
  }
  {
#pragma unroll
    for (int i = 0; i < R::VT; ++i) {
      const int task = tid + kAttnThreads * i;
      if (task < R::VTASKS) {
        const int kq = task / C::CPR, ch = task % C::CPR;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = min(j0 + 4 * kq + jj, jmax);
          r.v[i][jj] = *(const u32x4_t*)(V + ((size_t)j * Hkv + g) * D + ch * C::EPC);
        }
      }
    }
  }
}

// LDS stores of a loaded fp32 tile: K row-major into Ks, V transposed into Vt.
template <bool BF16, int D, typename E>
__device__ __forceinline__ void kv_store(const KVRegs<BF16, D>& r, E* __restrict__ Ks,
                                         E* __restrict__ Vt, int tid) {
  using C = AttnCfg<BF16, D>;
  using R = KVRegs<BF16, D>;
#pragma unroll
  for (int i = 0; i < R::KT; ++i) {
    const int task = tid + kAttnThreads * i;
    const int row = task / C::CPR, ch = task % C::CPR;
    *(u32x4_t*)(Ks + row * C::KS + ch * C::EPC) = r.k[i];
  }
  {
#pragma unroll
    for (int i2 = 0; i2 < R::VT; ++i2) {
      const int task = tid + kAttnThreads * i2;
      if (task < R::VTASKS) {
        const int kq = task / C::CPR, ch = task % C::CPR;
        const u32x4_t* x = r.v[i2];
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
}

// Walks the key tiles of a work entry: the query tile's key-tile sequence is
// every ancestor segment's range (fully visible), nearest ancestor first, then
// the root's resumed context (cache rows, fully visible), then the tile's own
// range (tree-masked), 64 keys per tile; the entry covers tiles [kt0, kt1) of
// it. ph: 0 ancestors (segment a), 1 the context [c0, c1), 2 the own range;
// cx marks a range of cache rows.
struct TileIter {
  int a, j0, hi, left, ph, c0, c1;
  bool own, cx, done;
};

// Positions it at the start of the range of (ph, a), moving on past empty ones.
__device__ __forceinline__ void iter_range(TileIter& it, const AttnTile& tile,
                                           const int32_t* __restrict__ seg_start,
                                           const int32_t* __restrict__ seg_len) {
  if (it.ph == 0) {
    if (it.a >= 0) {
      it.j0 = seg_start[it.a];
      it.hi = it.j0 + seg_len[it.a];
      it.own = it.cx = false;
      return;
    }
    it.ph = 1;
  }
  if (it.ph == 1) {
    if (it.c1 > it.c0) {
      it.j0 = it.c0;
      it.hi = it.c1;
      it.own = false;
      it.cx = true;
      return;
    }
    it.ph = 2;
  }
  it.j0 = tile.own_lo;
  it.hi = tile.t1;
  it.own = true;
  it.cx = false;
}

__device__ __forceinline__ void iter_advance(TileIter& it, const AttnTile& tile,
                                             const int32_t* __restrict__ parent,
                                             const int32_t* __restrict__ seg_start,
                                             const int32_t* __restrict__ seg_len) {
  if (it.ph == 0)
    it.a = parent[it.a];
  else
    it.ph = 2;
  iter_range(it, tile, seg_start, seg_len);
}

// ctx_start / ctx_len: the blob's context arrays, or null (no context)
__device__ __forceinline__ void iter_init(TileIter& it, const AttnTile& tile,
                                          const int32_t* __restrict__ parent,
                                          const int32_t* __restrict__ seg_start,
                                          const int32_t* __restrict__ seg_len,
                                          const int32_t* __restrict__ ctx_start,
                                          const int32_t* __restrict__ ctx_len) {
  int skip = tile.kt0;
  it.left = tile.kt1 - tile.kt0;
  it.done = it.left <= 0;
  it.a = (tile.info & kTileAncMask) - 1;
  it.c0 = ctx_len ? ctx_start[tile.root] : 0;
  it.c1 = ctx_len ? it.c0 + ctx_len[tile.root] : 0;
  it.ph = 0;
  iter_range(it, tile, seg_start, seg_len);
  while (!it.own) {
    const int n = (it.hi - it.j0 + kAttnKeys - 1) / kAttnKeys;
    if (skip < n) break;
    skip -= n;
    iter_advance(it, tile, parent, seg_start, seg_len);
  }
  it.j0 += kAttnKeys * skip;
}

__device__ __forceinline__ void iter_next(TileIter& it, const AttnTile& tile,
                                          const int32_t* __restrict__ parent,
                                          const int32_t* __restrict__ seg_start,
                                          const int32_t* __restrict__ seg_len) {
  if (--it.left <= 0) {
    it.done = true;
    return;
  }
  it.j0 += kAttnKeys;
  if (it.j0 < it.hi) return;
  if (it.own) {
    it.done = true;
    return;
  }
  iter_advance(it, tile, parent, seg_start, seg_len);
}

// One workgroup of 8 waves per CU: two waves per SIMD, <= 256 VGPRs each.
template <bool BF16, int D, bool F8>
__global__ void __launch_bounds__(kAttnThreads, 1)
    fork_attn_kernel(const int32_t* __restrict__ blob, AttnArgs args) {
  using C = AttnCfg<BF16, D, F8>;
  using E = typename std::conditional<BF16, unsigned short, float>::type;
  using QF = typename std::conditional<BF16, bf16x8_t, float>::type;
  // bf16: three K/V tile buffers (static arrays, so the compiler can tell the
  // buffer being read from the ones being filled by DMA); fp32: one K tile in
  // lds0 and the transposed V tile in lds1.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[BF16 ? C::BUF_BYTES : 16];

  if (!blob_ok(blob, args.guard)) return;  // (before any other blob access; no counter touched)
  const int ntiles = blob[MH_NTILES];
  const int TT = blob[MH_TILE_TOKENS];
  const AttnTile* __restrict__ tiles = (const AttnTile*)(blob + blob[MH_OFF_TILES]);
  const int32_t* __restrict__ parent = blob + blob[MH_OFF_PARENT];
  const int32_t* __restrict__ seg_len = blob + blob[MH_OFF_SEGLEN];
  const int32_t* __restrict__ seg_start = blob + blob[MH_OFF_SEGSTART];
  const int32_t* __restrict__ tok_pos = blob + blob[MH_OFF_TOKPOS];
  // resumed contexts: only when the blob has any and the cache is given
  const bool has_ctx = args.kc != nullptr && blob[MH_NCTX] > 0;
  const int32_t* __restrict__ ctx_start = has_ctx ? blob + blob[MH_OFF_CTXSTART] : nullptr;
  const int32_t* __restrict__ ctx_len = has_ctx ? blob + blob[MH_OFF_CTXLEN] : nullptr;
  const E* __restrict__ Q = (const E*)args.q;
  const E* __restrict__ K = (const E*)args.k;
  const E* __restrict__ V = (const E*)args.v;
  const E* __restrict__ Kc = (const E*)args.kc;
  const E* __restrict__ Vc = (const E*)args.vc;
  E* __restrict__ O = (E*)args.o;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int H = args.H, Hkv = args.Hkv, G = args.G;
  const int nitems = ntiles * Hkv;
  __shared__ int s_item;

  // Work items (most expensive first) are handed out dynamically, per XCD:
  // workgroups are dispatched round-robin over the 8 XCDs (the grid is a
  // multiple of 8), and the workgroups of XCD x take items x, x + 8, x + 16,
  // ... from that XCD's counter in the blob. A workgroup that finishes early
  // takes the next item, while each XCD keeps to the kv heads g = item mod Hkv
  // it started with, so their keys and values stay in its L2. The counters are
  // zero when the blob is built; the last workgroup to run out of work resets
  // them for the next launch.
  // The first item of a workgroup is static (item blockIdx.x: the XCD's
  // counter starts past the first items of its workgroups), so no workgroup
  // waits on a contended counter at the start. The next item is requested
  // when the current item's last key tile starts, so the request's latency
  // is hidden behind that tile's compute while the assignment stays dynamic.
  const int xcd = blockIdx.x & (kNumXcd - 1);
  const int per_xcd = gridDim.x / kNumXcd;
  // quotients by G of row indices < 256 (G <= 128): (n + 1/2) / G in fp32 is
  // off by far less than 1 / (2 G), so truncation gives the exact quotient
  const float inv_g = 1.f / (float)G;
  auto div_g = [&](int n) { return (int)(((float)n + 0.5f) * inv_g); };

  // The current item's tile (uniform across the workgroup: scalar registers)
  // and kv head; the next item's are loaded, and its first key/value tile's
  // DMA issued, while the current item's output is stored.
  AttnTile tile;
  int g = 0;
  auto load_tile = [&](int itm) {
    const int tix = itm / Hkv;
    g = itm - tix * Hkv;
    tile.t0 = __builtin_amdgcn_readfirstlane(tiles[tix].t0);
    tile.t1 = __builtin_amdgcn_readfirstlane(tiles[tix].t1);
    tile.own_lo = __builtin_amdgcn_readfirstlane(tiles[tix].own_lo);
    tile.info = __builtin_amdgcn_readfirstlane(tiles[tix].info);
    tile.kt0 = __builtin_amdgcn_readfirstlane(tiles[tix].kt0);
    tile.kt1 = __builtin_amdgcn_readfirstlane(tiles[tix].kt1);
    tile.slot = __builtin_amdgcn_readfirstlane(tiles[tix].slot);
    tile.root = __builtin_amdgcn_readfirstlane(tiles[tix].root);
  };
  TileIter it;
  // bf16 key/value tiles in flight: DMA of the iterator's next tile into a
  // buffer, with the tile's range kept per buffer slot
  int pj[3], ph[3];
  bool po[3];
  int nq = 0;  // tiles issued and not yet computed
  auto issue = [&](unsigned char* buf, int slot) {
    if (it.done) return;
    pj[slot] = it.j0;
    ph[slot] = it.hi;
    po[slot] = it.own;
    if constexpr (F8)
      kv_dma_f8<D>(buf, (const unsigned char*)args.k, args.ks, V, it.j0, it.hi - 1, g, Hkv, wave, lane);
    else if constexpr (BF16)
      kv_dma<D>(buf, it.cx ? Kc : K, it.cx ? Vc : V, it.j0, it.hi - 1, g, Hkv, wave, lane);
    ++nq;
    iter_next(it, tile, parent, seg_start, seg_len);
  };
  auto start_item = [&](int itm) {
    load_tile(itm);
    iter_init(it, tile, parent, seg_start, seg_len, ctx_start, ctx_len);
    if constexpr (BF16) issue(lds2, 2);  // an item's first tile goes to lds2
  };

  int item = blockIdx.x;
  if (item < nitems) start_item(item);
  for (;;) {
    if (item >= nitems) break;
    bool requested = false;
    int nxt = 0;  // thread 0: the XCD counter's value for the next item
    auto request_next = [&]() {
      if (!requested) {
        requested = true;
        if (tid == 0) nxt = atomicAdd(args.ctr + xcd, 1);
      }
    };

    // this lane's query row (rows past the tile are clamped and not stored)
    // per item, from the thread id: the row math is recomputed rather than
    // kept in registers (or spilled) across the key loop
    int tt = (int)threadIdx.x;
    asm volatile("" : "+v"(tt));
    const int r = (tt >> 6) * 32 + (tt & 31);
    const int tl = div_g(r), hg = r - tl * G;
    const bool valid = tl < TT && tile.t0 + tl < tile.t1;
    const int t_row = valid ? tile.t0 + tl : tile.t1 - 1;
    const int h = g * G + (valid ? hg : 0);
    const int lo_row = t_row - tok_pos[t_row];
    // a wave whose 32 rows all lie past the tile's tokens (a partial tile)
    // skips the arithmetic of the key loop: its rows are never stored, and it
    // still takes part in every barrier and key/value load. Rows map to tokens
    // in order, so the wave's first row decides; the test is scalar.
    const int wv_first = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) * 32;
    const int ntok = tile.t1 - tile.t0 < TT ? tile.t1 - tile.t0 : TT;
    const bool wave_live = __builtin_amdgcn_readfirstlane(div_g(wv_first)) < ntok;

    // F8: this lane's 32 bytes of each 64-wide k-step of its q row (A and B
    // of the FP8 product hold the same d indices at the same byte places), and
    // the row's scale folded into the softmax factor c
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    i32x8_t qf8[F8 ? D / 64 : 1];
    float csc = args.scale_log2;
    if constexpr (F8) {
      int hq = hi;
      asm volatile("" : "+v"(hq));
      const unsigned char* qrow = (const unsigned char*)args.q + ((size_t)t_row * H + h) * D;
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks) {
        const u32x4_t lo = *(const u32x4_t*)(qrow + 64 * ks + 32 * hq);
        const u32x4_t hi4 = *(const u32x4_t*)(qrow + 64 * ks + 32 * hq + 16);
        qf8[ks] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
      }
      csc = args.qs[(size_t)t_row * H + h] * args.scale_log2;
    }
    QF qf[F8 ? 1 : C::NKF];
    if constexpr (!F8) {
      int hq = hi;
      asm volatile("" : "+v"(hq));  // (as r above: no 64-bit base + hi offset kept across items)
      const E* qrow = Q + ((size_t)t_row * H + h) * D;
#pragma unroll
      for (int ks = 0; ks < C::NKF; ++ks) {
        if constexpr (BF16)
          qf[ks] = *(const bf16x8_t*)(qrow + 16 * ks + 8 * hq);
        else
          qf[ks] = qrow[2 * ks + hq];
      }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

    // compute one staged 64-key tile of range [j0, hi_); own == tree-masked own range
    auto kv_compute = [&](const E* __restrict__ Ks, const E* __restrict__ Vt, int j0, int hi_, bool own) {
      // The 64-key tile is processed as two 32-key halves, software-pipelined
      // so that MFMA work and softmax VALU work of different halves sit in the
      // same scheduling group: QK(0) | QK(1) + softmax(0) | PV(0) + softmax(1)
      // | PV(1). With both waves of a SIMD in step, this is what keeps the
      // matrix core busy while the scores are exponentiated.
      const bool need_mask = own ? ((tile.info & kTileMulti) != 0 || j0 + kAttnKeys > tile.t0)
                                 : (j0 + kAttnKeys > hi_);
      f32x16_t s[2];
      auto qk = [&](int b) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[b][i] = 0.f;
        if constexpr (F8) {
          // key row 32 b + l32: 32 bytes (16-byte chunks 4 ks + 2 hi, + 1) per k-step
          const unsigned char* K8 = (const unsigned char*)Ks;
          const int kr = 32 * b + l32;
#pragma unroll
          for (int ks = 0; ks < D / 64; ++ks) {
            const u32x4_t lo = *(const u32x4_t*)(K8 + kr * D + 16 * k8_chunk_pos(kr, 4 * ks + 2 * hi));
            const u32x4_t hi4 = *(const u32x4_t*)(K8 + kr * D + 16 * k8_chunk_pos(kr, 4 * ks + 2 * hi + 1));
            const i32x8_t a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
            // formats 0 (E4M3) for both operands, unit block scales (E8M0 127)
            s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[ks], s[b], 0, 0, 0, 127, 0, 127);
          }
          // the keys' scales (this lane's 16 keys: 32 b + 8 q + 4 hi + r)
          const float* kss = (const float*)(K8 + C::KS_OFF);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t k4 = *(const f32x4_t*)(kss + 32 * b + 8 * q + 4 * hi);
#pragma unroll
            for (int r = 0; r < 4; ++r) s[b][4 * q + r] *= k4[r];
          }
          return;
        }
#pragma unroll
        for (int ks = 0; ks < C::NKF; ++ks) {
          if constexpr (BF16) {
            const int kr = 32 * b + l32;
            const bf16x8_t a = *(const bf16x8_t*)(Ks + kr * D + 8 * k_chunk_pos<D / 8>(kr, 2 * ks + hi));
            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[b], 0, 0, 0);
          } else {
            const float a = Ks[(32 * b + l32) * C::KS + 2 * ks + hi];
            s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[ks], s[b], 0, 0, 0);
          }
        }
      };
      // Online softmax in log2 units, p = exp2(s * c - m) with c = scale * log2(e),
      // one 32-key half at a time, in two parts. sm_max: tree mask, row max and
      // the running-max update (a lane raises its max m only when the half's
      // max exceeds it by more than 8, a factor of 256; otherwise the stale max
      // is kept, which is exact since numerator and denominator share m, keeps
      // p <= 256 and makes rescaling rare). sm_exp: the exponentials, row sums
      // and bf16 packing, free of branches so that they can share a
      // scheduling group with MFMAs.
      float alpha[2];
      bool grew[2];
      auto sm_max = [&](int b) {
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = j0 + 32 * b + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool vis = (j < hi_) & (!own | ((j >= lo_row) & (j <= t_row)));
            s[b][i] = vis ? s[b][i] : -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
        const LanePair mp = lane_pair(mx);
        mx = fmaxf(mp.a, mp.b) * csc;
        const bool grow = mx > m_run + 8.f;
        alpha[b] = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
        m_run = grow ? mx : m_run;
        grew[b] = __any(grow);
        l_run *= alpha[b];
      };
      typename std::conditional<BF16, bf16x8_t, float>::type pb[2][2];
      auto sm_exp = [&](int b) {
        const float mneg = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[b][i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], csc, mneg));
        if constexpr (BF16) {
          // bf16 P (the operand of the value product); the row sum adds these
          // rounded weights, two per dot instruction (exact products by 1,
          // fp32 sums), so the normaliser matches the weights applied
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
          float ps[2] = {0.f, 0.f};
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) pb[b][hf][jj] = (__bf16)s[b][8 * hf + jj];
#pragma unroll
            for (int q = 0; q < 4; ++q)
            {
              const bf16x2_t pr = {pb[b][hf][2 * q], pb[b][hf][2 * q + 1]};
              ps[hf] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ps[hf], false);
            }
          }
          l_run += ps[0] + ps[1];
        } else {
          float psum = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) psum += s[b][i];
          l_run += psum;
        }
      };
      auto rescale = [&](int b) {
        if (grew[b]) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha[b];
        }
      };
      // O^T += V^T P^T for one 32-key half
      auto pv = [&](int b) {
        if constexpr (BF16) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            // A = V^T fragments by transposing LDS reads: within each group of
            // 16 lanes, lane L points at key row (L / 4) of a 4-key block and
            // d column 4 (L % 4); lane i of the group receives the 4 keys at
            // d = d0 + i. Two reads give keys {+0..3} and {+8..11}, matching
            // the key order of the P^T fragment.
            const int g16 = lane >> 4, L16 = lane & 15;
            const int krow = 32 * b + 16 * hf + 4 * hi + (L16 >> 2);
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
              const int col = 32 * db + 16 * (g16 & 1) + 4 * (L16 & 3);
              // col = 8 * chunk + 4 * half; krow and krow + 8 agree mod 4
              const int vpos = 8 * v_chunk_pos<D / 8>(krow, col >> 3) + (col & 7);
              const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + krow * D + vpos));
              const s16x4_t hi4 =
                  __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + (krow + 8) * D + vpos));
              typedef short s16x8_t __attribute__((ext_vector_type(8)));
              const s16x8_t w8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
              const bf16x8_t va = __builtin_bit_cast(bf16x8_t, w8);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[b][hf], oacc[db], 0, 0, 0);
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
      };
      // Pipeline over the two halves. The running max may rise at either half:
      // half 0's rise rescales the accumulators before anything of this tile is
      // added; half 1's rise rescales them after half 0's products are in, so
      // that both halves' products end up relative to the final max. Scheduling
      // groups (masks: 0x008 MFMA, 0x002 VALU, 0x100 LDS read) alternate one
      // MFMA with a run of VALU instructions in the two mixed groups.
      qk(0);
      __builtin_amdgcn_sched_barrier(0);
      sm_max(0);
      rescale(0);
      __builtin_amdgcn_sched_barrier(0);
      qk(1);
      sm_exp(0);
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < C::NKF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      sm_max(1);
      __builtin_amdgcn_sched_barrier(0);
      pv(0);
      sm_exp(1);
      if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 2 * C::NDB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      rescale(1);
      pv(1);
    };

    if constexpr (BF16) {
      // Software pipeline over three LDS buffers: the DMAs of tiles i+1 and
      // i+2 are in flight while tile i computes. Per tile: wait for this
      // wave's DMA of tile i (its DMA of tile i+1 may stay in flight), one
      // barrier (every wave's DMA of tile i landed; every wave is done with
      // tile i-1, whose buffer tile i+2 then fills), issue that DMA, compute.
      // Tiles cycle through lds2, lds0, lds1 (tile 0 was issued into lds2
      // while the previous item stored its output); the loop is unrolled by
      // three so that each step reads and fills fixed buffers.
      // per wave and tile: K and V blocks (FP8: one K block, two V blocks, one dword load of key scales)
      constexpr int DMA_PER_TILE = F8 ? 4 : 2 * (kAttnKeys * D * 2 / 1024) / (kAttnThreads / 64);
      static_assert(DMA_PER_TILE < 16, "vmcnt field");
      __syncthreads();  // the previous item's output rows staged in lds0 / lds1 are read
      issue(lds0, 0);
      auto step = [&](unsigned char* cur, int slot, unsigned char* fill, int fslot) {
        if (nq > 1)
          __builtin_amdgcn_s_waitcnt(0x0f70 | DMA_PER_TILE);  // vmcnt: tile i landed, i+1 may fly
        else
          __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        --nq;
        // the last tile: every DMA of this wave has landed, so the request
        // (a returning atomic, counted with them) delays no tile wait
        if (nq == 0 && it.done) request_next();
        issue(fill, fslot);
        if (wave_live) kv_compute((const E*)cur, (const E*)(cur + C::V_OFF), pj[slot], ph[slot], po[slot]);
      };
      while (nq > 0) {
        step(lds2, 2, lds1, 1);
        if (nq == 0) break;
        step(lds0, 0, lds2, 2);
        if (nq == 0) break;
        step(lds1, 1, lds0, 0);
      }
    } else {
      // fp32: registers hold tile i+1 while tile i computes
      E* Ks = (E*)lds0;
      E* Vt = (E*)lds1;
      KVRegs<BF16, D> rg;
      kv_load<BF16, D, E>(rg, it.cx ? Kc : K, it.cx ? Vc : V, it.j0, it.hi - 1, g, Hkv, tid);
      while (!it.done) {
        const int j0 = it.j0, hi_ = it.hi;
        const bool own = it.own;
        __syncthreads();  // every wave is done with the previous tile
        kv_store<BF16, D, E>(rg, Ks, Vt, tid);
        __syncthreads();
        iter_next(it, tile, parent, seg_start, seg_len);
        if (!it.done)
          kv_load<BF16, D, E>(rg, it.cx ? Kc : K, it.cx ? Vc : V, it.j0, it.hi - 1, g, Hkv, tid);
        else
          request_next();
        if (wave_live) kv_compute(Ks, Vt, j0, hi_, own);
      }
    }

    // the next item: requested at the last tile, long returned by now; written
    // before this item's stores are issued, so reading it waits for nothing
    // (every thread read the current item before the first tile's barrier)
    request_next();  // (an item whose tiles never triggered it)
    if (tid == 0) s_item = (nxt + per_xcd) * kNumXcd + xcd;
    // s_item is visible, and every wave is done with the last key/value tile
    // (its buffers are reused below); this barrier waits for no store
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int next_item = s_item;
    // this item's tile fields for the stores below; then the next item's tile
    // record and first DMA, in flight while this item's output is stored
    const int f_t0 = tile.t0, f_t1 = tile.t1, f_slot = tile.slot, f_g = g;
    if (next_item < nitems) start_item(next_item);

    // finalize: normalise; whole tiles store the output, parts of a split tile
    // store their normalised rows (output dtype) and log-sum-exps into the
    // tile's slot for the merge pass
    const LanePair lp = lane_pair(l_run);
    const float l_tot = lp.a + lp.b;  // (the same sum in both lanes of the row)
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_row = l_tot > 0.f ? m_run * 0.6931471805599453f + __logf(l_tot) : -INFINITY;
    constexpr size_t SLOT = (size_t)kAttnRows * D * sizeof(E) + (size_t)kAttnRows * 4;
    unsigned char* part = f_slot >= 0 ? args.ws + ((size_t)f_slot * Hkv + f_g) * SLOT : nullptr;
    if (valid && hi == 0) {
      if (f_slot >= 0)
        ((float*)((E*)part + kAttnRows * D))[r] = lse_row;
      else if (args.lse)
        args.lse[(size_t)t_row * H + h] = lse_row;
    }
    if constexpr (BF16) {
      // A lane's accumulators hold 4-element pieces of one row (the piece at d
      // = 32 db + 8 rq + 4 hi), so storing them directly writes 8 bytes into
      // each of 32 rows per instruction. Instead each wave stages its 32 rows
      // in lds0 (waves 0-3) or lds1 (waves 4-7), the 16-byte chunk c of row r
      // at position c ^ (r mod LPR) against bank conflicts, and stores whole
      // rows, 16 bytes per lane.
      constexpr int ORB = D * 2;       // bytes per staged row
      constexpr int LPR = ORB / 16;    // lanes (16-byte chunks) per row
      constexpr int RPI = 64 / LPR;    // rows per store instruction
      constexpr int NST = 32 / RPI;    // store instructions per wave
      static_assert(4 * 32 * ORB <= C::BUF_BYTES, "four waves' rows per buffer");
      // lane-derived indices are recomputed here rather than hoisted out of
      // the item loop, where they would hold registers through the key loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      unsigned char* stg = (wv < 4 ? lds0 : lds1) + (wv & 3) * 32 * ORB;
      const int srow = ln & 31;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          bf16x2_t p0, p1;
          p0[0] = (__bf16)(oacc[db][4 * rq + 0] * inv);
          p0[1] = (__bf16)(oacc[db][4 * rq + 1] * inv);
          p1[0] = (__bf16)(oacc[db][4 * rq + 2] * inv);
          p1[1] = (__bf16)(oacc[db][4 * rq + 3] * inv);
          uint2 pk;
          pk.x = __builtin_bit_cast(unsigned, p0);
          pk.y = __builtin_bit_cast(unsigned, p1);
          const int ch = 4 * db + rq;  // 16-byte chunk of the row
          *(uint2*)(stg + srow * ORB + 16 * (ch ^ (srow % LPR)) + 8 * (ln >> 5)) = pk;
        }
      // all reads first (one LDS round trip), then the stores
      u32x4_t v[NST];
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const int rl = k * RPI + ln / LPR;
        v[k] = *(const u32x4_t*)(stg + rl * ORB + 16 * ((ln % LPR) ^ (rl % LPR)));
      }
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const int rr = wv * 32 + k * RPI + ln / LPR;
        const int tl2 = div_g(rr), hg2 = rr - tl2 * G;
        if (tl2 < TT && f_t0 + tl2 < f_t1) {
          E* dst = f_slot >= 0 ? (E*)part + rr * D : O + ((size_t)(f_t0 + tl2) * H + f_g * G + hg2) * D;
          *(u32x4_t*)(dst + 8 * (ln % LPR)) = v[k];
        }
      }
    } else {
      if (valid) {
        E* orow = f_slot >= 0 ? (E*)part + r * D : O + ((size_t)t_row * H + h) * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * db + 8 * rq + 4 * hi;
            *(float4*)(orow + d0) = make_float4(oacc[db][4 * rq + 0] * inv, oacc[db][4 * rq + 1] * inv,
                                                oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv);
          }
      }
    }
    item = next_item;
  }
  if (tid == 0 && atomicAdd(args.ctr + kNumXcd, 1) == (int)gridDim.x - 1) {
    // every other workgroup has taken its last item: reset for the next launch
    for (int x = 0; x <= kNumXcd; ++x) atomicExch(args.ctr + x, 0);
  }
}

// Combines the parts of split query tiles: for each row,
// o = sum_p exp(lse_p - lse) o_p with lse = log sum_p exp(lse_p).
// A work item is (split tile, kv head, group of 16 rows); 16 threads share a
// row and each combines D / 16 consecutive columns of it. Every load of an
// item (each part's log-sum-exp and columns) is issued before any of them is
// used, so an item costs one memory round trip.
constexpr int kMergeRows = 16;
template <bool BF16, int D>
__global__ void __launch_bounds__(256) fork_attn_merge_kernel(const int32_t* __restrict__ blob, AttnArgs args) {
  using E = typename std::conditional<BF16, unsigned short, float>::type;
  constexpr size_t SLOT = (size_t)kAttnRows * D * sizeof(E) + (size_t)kAttnRows * 4;  // bytes per partial slot
  constexpr int NRG = kAttnRows / kMergeRows;  // row groups per tile
  constexpr int CPT = D / 16;                  // columns per thread
  constexpr int NDW = CPT * (int)sizeof(E) / 4;  // their dwords
  static_assert(NDW == 2 || NDW % 4 == 0, "8-byte or whole 16-byte loads");
  if (!blob_ok(blob, args.guard)) return;
  const int nmerge = blob[MH_NMERGE];
  const int TT = blob[MH_TILE_TOKENS];
  const AttnMerge* __restrict__ merges = (const AttnMerge*)(blob + blob[MH_OFF_MERGE]);
  const int H = args.H, Hkv = args.Hkv, G = args.G;
  const int rr = threadIdx.x >> 4, cq = threadIdx.x & 15;
  for (int item = blockIdx.x; item < nmerge * Hkv * NRG; item += gridDim.x) {
    const int rg = item % NRG, mg = item / NRG;
    const int mi = mg / Hkv, g = mg - mi * Hkv;
    const int t0 = merges[mi].t0, t1 = merges[mi].t1, np = merges[mi].nparts, s0 = merges[mi].slot0;
    const int r = kMergeRows * rg + rr;
    const int tl = r / G, hg = r - tl * G;
    if (tl >= TT || t0 + tl >= t1) continue;
    const unsigned char* part0 = args.ws + ((size_t)s0 * Hkv + g) * SLOT;
    const size_t pstride = (size_t)Hkv * SLOT;
    float lp[kMaxSplit];
    unsigned wv[kMaxSplit][NDW];
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p) {
      lp[p] = -INFINITY;
      if (p < np) {
        const unsigned char* base = part0 + p * pstride;
        lp[p] = ((const float*)(base + (size_t)kAttnRows * D * sizeof(E)))[r];
        const unsigned* src = (const unsigned*)((const E*)base + (size_t)r * D + CPT * cq);
        if constexpr (NDW == 2) {
          const uint2 u = *(const uint2*)src;
          wv[p][0] = u.x;
          wv[p][1] = u.y;
        } else {
#pragma unroll
          for (int q = 0; q < NDW; q += 4) {
            const uint4 u = *(const uint4*)(src + q);
            wv[p][q] = u.x;
            wv[p][q + 1] = u.y;
            wv[p][q + 2] = u.z;
            wv[p][q + 3] = u.w;
          }
        }
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p) m = fmaxf(m, lp[p]);
    float den = 0.f;
    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p) {
      if (p < np) {
        const float wgt = lp[p] == -INFINITY ? 0.f : __expf(lp[p] - m);
        den += wgt;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          const float x = BF16 ? __uint_as_float((j & 1) ? (wv[p][j >> 1] & 0xffff0000u) : (wv[p][j >> 1] << 16))
                               : __uint_as_float(wv[p][j]);
          acc[j] += wgt * x;
        }
      }
    }
    const float inv = 1.f / den;
    const int t = t0 + tl, h = g * G + hg;
    unsigned* orow = (unsigned*)((E*)args.o + ((size_t)t * H + h) * D + CPT * cq);
    unsigned ov[NDW];
    if constexpr (BF16) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int q = 0; q < NDW; ++q) {
        bf16x2_t pr;
        pr[0] = (__bf16)(acc[2 * q] * inv);
        pr[1] = (__bf16)(acc[2 * q + 1] * inv);
        ov[q] = __builtin_bit_cast(unsigned, pr);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NDW; ++q) ov[q] = __float_as_uint(acc[q] * inv);
    }
    if constexpr (NDW == 2) {
      *(uint2*)orow = make_uint2(ov[0], ov[1]);
    } else {
#pragma unroll
      for (int q = 0; q < NDW; q += 4) *(uint4*)(orow + q) = make_uint4(ov[q], ov[q + 1], ov[q + 2], ov[q + 3]);
    }
    if (args.lse && cq == 0) args.lse[(size_t)t * H + h] = m + __logf(den);
  }
}

template <bool BF16, int D, bool F8 = false>
fork_status launch_one(const fork_meta* m, const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fork_attn_kernel<BF16, D, F8>), dim3(grid), dim3(kAttnThreads), 0, stream, a.blob, a);
  FORK_HIP_CHECK(hipGetLastError());
  // merge pass for split tiles: under capture whenever splitting is possible,
  // otherwise only when this tree has split tiles
  const bool cap = stream_capturing(stream);
  if (m->caps.kv_heads > 0 && (cap || m->num_attn_merges > 0)) {
    int mgrid = 4 * device_cu_count();
    if (!cap) mgrid = std::min(mgrid, m->num_attn_merges * a.Hkv * (kAttnRows / kMergeRows));
    hipLaunchKernelGGL((fork_attn_merge_kernel<BF16, D>), dim3(mgrid), dim3(256), 0, stream, a.blob, a);
    FORK_HIP_CHECK(hipGetLastError());
  }
  return FORK_OK;
}

// Partial results of split query tiles for fork_attn_forward_noalloc: a
// file-scope device array, one copy per GPU. Host code never passes the
// array's name to a kernel (on the host it only names the symbol): it takes
// each device's address once through hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[FORK_ATTN_SCRATCH_BYTES];

}  // namespace

fork_status attn_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  FORK_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(FORK_E_UNSUPPORTED, "device ordinal %d (at most 64 devices)", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    FORK_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(FORK_E_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return FORK_OK;
}

size_t attn_workspace_bytes(const fork_caps& c, int D, fork_dtype dt) {
  return c.kv_heads > 0 ? (size_t)kMaxPartSlots * attn_slot_bytes(D, dt) : 0;
}

fork_status launch_attention(const fork_meta* m, const void* q, const void* k, const void* v,
                             const void* kc, const void* vc, void* o, float* lse, int H, int Hkv, int D,
                             float scale, fork_dtype dt, void* ws, hipStream_t stream) {
  return launch_attention_any(m, q, nullptr, k, nullptr, v, kc, vc, o, lse, H, Hkv, D, scale, dt, ws, stream);
}

fork_status launch_attention_any(const fork_meta* m, const void* q, const float* qs, const void* k, const float* ks,
                                 const void* v, const void* kc, const void* vc, void* o, float* lse, int H, int Hkv,
                                 int D, float scale, fork_dtype dt, void* ws, hipStream_t stream) {
  AttnArgs a;
  a.qs = qs;
  a.ks = ks;
  a.blob = (const int32_t*)m->dev;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = kc;
  a.vc = vc;
  a.o = o;
  a.lse = lse;
  a.ws = (unsigned char*)ws;
  a.ctr = (int32_t*)m->dev + kAttnCtrWord;
  a.guard = blob_guard(m->caps);
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  const float sc = scale > 0.f ? scale : 1.f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  // Persistent grid: one workgroup per CU. Under capture the tree can change
  // between replays, so the grid must not depend on the current tile count.
  int grid = device_cu_count();
  if (!stream_capturing(stream)) {
    const long long items = (long long)m->num_attn_tiles * Hkv;
    if (items < grid) grid = (int)(items > 0 ? items : 1);
  }
  grid = (grid + kNumXcd - 1) / kNumXcd * kNumXcd;  // whole rounds over the XCDs
  if (qs) return launch_one<true, 128, true>(m, a, grid, stream);  // FP8 scores (checked by the caller)
  if (dt == FORK_BF16)
    return D == 128 ? launch_one<true, 128>(m, a, grid, stream) : launch_one<true, 64>(m, a, grid, stream);
  return D == 128 ? launch_one<false, 128>(m, a, grid, stream) : launch_one<false, 64>(m, a, grid, stream);
}

}  // namespace fork
