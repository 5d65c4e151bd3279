// Internal definitions shared by the host code and the HIP kernels of the
// ForkAttention library: the layout of the metadata blob, launch helpers and
// the error channel. Nothing here is part of the public C ABI (include/fork.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fork.h"

namespace fork {

// ---------------------------------------------------------------------------
// Metadata blob. The blob starts with MH_WORDS int32 header words; arrays are
// addressed by word offsets stored in the header, so kernels recorded in a
// graph find the arrays of whatever tree was built last. The header and the
// host-built arrays form one contiguous "upload" region copied in a single
// hipMemcpyAsync; the per-token arrays follow at offsets fixed by the
// capacities and are written on the device.
enum MetaHeader : int {
  MH_MAGIC = 0,
  MH_T,            // tokens
  MH_S,            // segments
  MH_R,            // roots
  MH_MAXDEPTH,     // deepest segment depth
  MH_NTILES,       // attention query tiles
  MH_NCHUNKS,      // Gated DeltaNet chunks
  MH_TILE_TOKENS,  // tokens per attention query tile
  MH_GQA,          // H / Hkv the tiles were cut for
  MH_OFF_PARENT,   // [S] parent segment or -1
  MH_OFF_SEGLEN,   // [S]
  MH_OFF_SEGSTART, // [S] first token
  MH_OFF_DEPTH,    // [S]
  MH_OFF_ROOT,     // [S] root segment
  MH_OFF_ROOTORD,  // [S] ordinal of the segment among roots (-1 for non-roots)
  MH_OFF_ANCLEN,   // [S] tokens in ancestors
  MH_OFF_FIRSTCHILD,  // [S] lowest-index child or -1
  MH_OFF_CHUNKBASE,   // [S] index of the segment's first chunk
  MH_OFF_LEVELOFF,    // [MAXDEPTH + 2] start of each depth in LEVELSEG
  MH_OFF_LEVELSEG,    // [S] segments by depth, longest first within a depth
  MH_OFF_CHUNKS,      // [NCHUNKS] int2 {first token, length}
  MH_OFF_TILES,       // [NTILES] AttnTile work entries, most expensive first
  MH_OFF_TOKSEG,      // [T] (device-written)
  MH_OFF_TOKPOS,      // [T] (device-written)
  MH_OFF_TOKISO,      // [T] (device-written)
  MH_UPLOAD_WORDS,    // size of the upload region in words
  MH_NMERGE,          // split query tiles (merge groups)
  MH_OFF_MERGE,       // [NMERGE] AttnMerge
  MH_NPARTS,          // partial-result slots used by split tiles (per kv head)
  MH_KV_HEADS,        // kv heads the split plan assumed (0: no splitting)
  MH_OFF_LEVELLONG,   // [MAXDEPTH + 1] segments longer than one GDN chunk at each depth (they lead its LEVELSEG list)
  MH_OFF_CTXSTART,    // [S] first key/value cache row of a root's resumed context (0 if none)
  MH_OFF_CTXLEN,      // [S] cache rows of a root's resumed context (0 for non-roots)
  MH_NCTX,            // roots with a nonempty context
  MH_OFF_GDNREC,      // [S x kGdnRecWords] Gated DeltaNet scan items in LEVELSEG order (GdnRec)
  MH_OFF_GDNPACK,     // [<= S x kGdnRecWords] scan items with leaf siblings packed (GdnRec), by depth
  MH_OFF_PACKOFF,     // [MAXDEPTH + 2] start of each depth in GDNPACK
  MH_WORDS = 64
};
// Header word 57 is the device error word (FORK_DEVERR_* bits, fork_meta_check).
constexpr int kErrWord = 57;
// Header words 48..56 hold the attention work counters: the next work item of
// each of the 8 XCDs (workgroup id mod 8), then the number of workgroups that
// found no more work. They are zero in a freshly built blob and the kernel
// leaves them zero.
constexpr int kAttnCtrWord = 48;
constexpr int kNumXcd = 8;
// Header words 58..59 hold the Gated DeltaNet scan's work counters (the next
// work item of a depth's launch, then the number of workgroups that found no
// more work), zero between launches like the attention counters.
constexpr int kGdnCtrWord = 58;
static_assert(kAttnCtrWord > MH_OFF_PACKOFF && kAttnCtrWord + kNumXcd < kErrWord && kErrWord < kGdnCtrWord &&
                  kGdnCtrWord + 2 <= MH_WORDS,
              "counter and error words inside the header, past the plan's words");


constexpr int32_t kMetaMagic = 0x464B4D31;  // "FKM1"
constexpr int kChunk = 64;                  // Gated DeltaNet chunk length
constexpr int kAttnRows = 256;              // query rows (token x GQA head) per attention tile
constexpr int kAttnKeys = 64;               // keys per staged key/value tile
constexpr int kMaxDepthCap = 4096;
// A Gated DeltaNet scan item's record, so that a scan workgroup learns
// everything about its next item from one load: its first segment, first
// token and length, the slot its start state is copied from (the first child
// of its parent, which holds the parent's end state; -1 - root ordinal for a
// root), the first child (-1 for a leaf) and the number of segments. GDNREC
// holds one record per segment (nsib = 1) in the level order; GDNPACK the
// same items except that runs of consecutive leaf siblings of at most one
// chunk (kChunk tokens) in total share one record: they start from the same
// state and no end state of theirs is carried on, so one chunk computes them
// all (used when no end states are requested). Each depth of GDNPACK is
// sorted longest first (stable), so its segments longer than a chunk lead it
// in the same order as in LEVELSEG. Padded to 8 words (two 16-byte loads).
struct GdnRec {
  int32_t seg, start, len, src, first_child, nsib, pad0, pad1;
};
constexpr int kGdnRecWords = 8;
static_assert(sizeof(GdnRec) == 4 * kGdnRecWords, "GdnRec layout");
// Split plan for query tiles with long key ranges: the number of shares the
// total work is cut into (the part size is total / kAttnSlots key tiles;
// about 1.6 parts per resident workgroup on a 256-CU MI355X, measured best
// on the one-request tree), the smallest part (in 64-key tiles), the most
// parts per tile, and the partial-result slots the workspace holds (parts x
// kv heads).
constexpr int kAttnSlots = 416;
constexpr int kMinPartTiles = 4;
constexpr int kMaxSplit = 16;
constexpr int kMaxPartSlots = 1024;

// One attention work entry: query tokens [t0, t1) of one or several
// consecutive sibling segments, and the part [kt0, kt1) of its key-tile
// sequence (ancestor segments nearest first, then the own range, 64 keys per
// tile) it covers. own_lo is the first token of t0's segment; info packs the
// segment whose ancestor path (itself included) every row sees in full
// (anc + 1, 0 for a root tile) in bits 0..29 and "tile spans several
// segments" in bit 30. slot is -1 for a whole tile (written straight to the
// output) or the partial-result slot of a split tile's part. root is the
// root segment of the tile's rows: its resumed context (if any) follows the
// ancestors in the key-tile sequence, before the own range.
struct AttnTile {
  int32_t t0, t1, own_lo, info;
  int32_t kt0, kt1, slot, root;
};
// A split query tile: its tokens and the `nparts` consecutive partial slots
// (from slot0) its parts wrote.
struct AttnMerge {
  int32_t t0, t1, nparts, slot0;
};
constexpr int32_t kTileMulti = 1 << 30;
constexpr int32_t kTileAncMask = (1 << 30) - 1;

struct BlobLayout {
  int64_t tile_cap, chunk_cap, merge_cap;
  int64_t upload_cap_words;  // capacity of the upload region (header included)
  int64_t tok_off_words;     // first per-token array
  int64_t total_words;
  int32_t tile_tokens;
};

// Tokens per attention tile for a GQA group size (each token brings G rows).
inline int32_t tile_tokens_for(int32_t gqa) { return gqa >= kAttnRows ? 1 : kAttnRows / gqa; }

inline BlobLayout blob_layout(const fork_caps& c) {
  BlobLayout L;
  L.tile_tokens = tile_tokens_for(c.gqa_group);
  // base tiles, plus at most kMaxPartSlots extra entries from splitting
  L.tile_cap = ((int64_t)c.t_cap + L.tile_tokens - 1) / L.tile_tokens + c.s_cap + kMaxPartSlots;
  L.chunk_cap = ((int64_t)c.t_cap + kChunk - 1) / kChunk + c.s_cap;
  L.merge_cap = kMaxPartSlots / 2;
  // header + 12 segment arrays + level offsets and long counts + 2 words per chunk + 8 per tile
  // + 4 per merge group + the scan items' records, each array aligned to 4 words
  L.upload_cap_words = MH_WORDS + 12 * ((int64_t)c.s_cap + 4) + 2 * (c.depth_cap + 2 + 4) +
                       2 * L.chunk_cap + 4 + 8 * L.tile_cap + 4 + 4 * L.merge_cap + 4 +
                       2 * (kGdnRecWords * (int64_t)c.s_cap + 4) + c.depth_cap + 2 + 4;
  L.upload_cap_words = (L.upload_cap_words + 63) / 64 * 64;
  L.tok_off_words = L.upload_cap_words;
  L.total_words = L.tok_off_words + 3 * (((int64_t)c.t_cap + 63) / 64 * 64);
  return L;
}

// What a launch assumes about the blob it reads: the capacities its grids and
// workspaces were sized for. Every kernel checks the blob's header against
// it before touching anything else (blob_ok), so a blob that was rebuilt with
// larger capacities, or overwritten, behind a recorded graph stops the
// kernel instead of overflowing a workspace.
struct BlobGuard {
  int32_t t_cap, s_cap, depth_cap, tile_cap, chunk_cap;
};
inline BlobGuard blob_guard(const fork_caps& c) {
  const BlobLayout L = blob_layout(c);
  BlobGuard g;
  g.t_cap = c.t_cap;
  g.s_cap = c.s_cap;
  g.depth_cap = c.depth_cap;
  g.tile_cap = (int32_t)L.tile_cap;
  g.chunk_cap = (int32_t)L.chunk_cap;
  return g;
}

// True when the blob's header fits the guard. Otherwise thread 0 of the
// workgroup sets the error bit in the header's error word (a vector atomic)
// and the caller returns at once. Header words are uniform (scalar loads).
__device__ __forceinline__ bool blob_ok(const int32_t* __restrict__ blob, const BlobGuard& g) {
  int err = 0;
  if (blob[MH_MAGIC] != kMetaMagic) {
    err = FORK_DEVERR_MAGIC;
  } else {
    const int T = blob[MH_T], S = blob[MH_S], d = blob[MH_MAXDEPTH];
    const int nt = blob[MH_NTILES], nc = blob[MH_NCHUNKS];
    if (T < 1 || T > g.t_cap || S < 1 || S > g.s_cap || d < 0 || d > g.depth_cap || nt < 0 ||
        nt > g.tile_cap || nc < 0 || nc > g.chunk_cap)
      err = FORK_DEVERR_CAPACITY;
  }
  if (err == 0) return true;
  if (threadIdx.x == 0 && threadIdx.y == 0) atomicOr((int*)blob + kErrWord, err);
  return false;
}

// ---------------------------------------------------------------------------
// Error channel (thread-local message, see fork_last_error).
void set_error(const char* fmt, ...);
fork_status fail(fork_status st, const char* fmt, ...);

#define FORK_HIP_CHECK(expr)                                                        \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return ::fork::fail(FORK_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Resident workgroups that fit the device at `per_cu` workgroups per compute unit.
int device_cu_count();

// True when `stream` is being captured into a graph.
bool stream_capturing(hipStream_t stream);

// Validates a descriptor against its blob.
fork_status check_meta(const fork_meta* m);

// Kernel launchers (defined with their kernels).
fork_status launch_meta_expand(const fork_meta* m, hipStream_t stream);
fork_status launch_dense_mask(const fork_meta* m, uint8_t* mask, hipStream_t stream);
// Bytes of one partial-result slot of a split query tile: kAttnRows x D
// normalised outputs in the output dtype, then kAttnRows fp32 log-sum-exps.
inline size_t attn_slot_bytes(int D, fork_dtype dt) {
  return (size_t)kAttnRows * D * (dt == FORK_BF16 ? 2 : 4) + (size_t)kAttnRows * 4;
}
size_t attn_workspace_bytes(const fork_caps& c, int D, fork_dtype dt);
// Device address of the current GPU's copy of the attention scratch array
// (FORK_ATTN_SCRATCH_BYTES), looked up once per device.
fork_status attn_scratch(void** ptr);
fork_status launch_attention(const fork_meta* m, const void* q, const void* k, const void* v,
                             const void* kc, const void* vc, void* o, float* lse, int H, int Hkv,
                             int D, float scale, fork_dtype dt, void* ws, hipStream_t stream);
// qs non-null: FP8 scores (q, k E4M3 codes with row scales qs [T, H], ks [T, Hkv]; v bf16; D 128)
fork_status launch_attention_any(const fork_meta* m, const void* q, const float* qs, const void* k, const float* ks,
                                 const void* v, const void* kc, const void* vc, void* o, float* lse, int H, int Hkv,
                                 int D, float scale, fork_dtype dt, void* ws, hipStream_t stream);
fork_status launch_rope(const fork_meta* m, const void* src, long long ld_src, void* dst, int nh, int D, float theta,
                        fork_dtype dt, hipStream_t stream);
fork_status launch_conv(const fork_meta* m, const void* x, const float* w, const float* bias,
                        const float* state, void* y, int C, int K, int act, fork_dtype dt,
                        hipStream_t stream);
fork_status launch_conv_split(const fork_meta* m, const void* x, const float* w, const float* bias,
                              const float* state, void* q, void* k, void* v, int H, int dk, int dv, int K, float eps,
                              fork_dtype dt, hipStream_t stream);
fork_status launch_gate(const fork_meta* m, const void* x, const void* g, long long ldg, const float* w, void* y,
                        int nh, int D, int mode, float eps, fork_dtype dt, hipStream_t stream);
fork_status launch_gdn_inputs(const fork_meta* m, const void* c, const void* ab, long long ld_ab, const float* a_log,
                              const float* dt_bias, void* q, void* k, void* v, float* a, float* b, int H, int dk,
                              int dv, float eps, fork_dtype dt, hipStream_t stream);
fork_status launch_linear(const void* x, const void* w, void* y, int M, int N, int K, int accumulate,
                          fork_dtype dt, hipStream_t stream);
fork_status launch_quantize_fp8(const void* x, void* q, float* scales, long long rows, int K, fork_dtype dt,
                                hipStream_t stream);
fork_status launch_readout(const fork_meta* m, const void* x, const float* w, int C, float* score, float* prob,
                           fork_dtype dt, hipStream_t stream);
fork_status launch_linear_fp8(const void* xq, const float* x_scale, const void* wq, const float* w_scale, void* y,
                              int M, int N, int K, int accumulate, hipStream_t stream);
size_t gdn_workspace_bytes(const fork_meta* m, int H, int dk, int dv);
fork_status launch_gdn(const fork_meta* m, const void* q, const void* k, const void* v,
                       const float* a, const float* b, const float* root_state, void* o,
                       float* seg_start_state, float* seg_final_state, int H, int dk, int dv,
                       float scale, fork_dtype dt, void* ws, size_t ws_bytes, hipStream_t stream);
fork_status launch_gdn_fp8(const fork_meta* m, const void* q8, const float* qs, const void* k8, const float* ks,
                           const void* v8, const float* vs, const float* a, const float* b, const float* root_state,
                           void* o, float* seg_start_state, float* seg_final_state, int H, float scale,
                           hipStream_t stream);

}  // namespace fork
