/*
 * fork.h - C ABI of the MI355X (gfx950) ForkAttention hot path.
 *
 * A decision request is a tree of token segments: a shared context prefix,
 * then child segments (candidate options or nested history branches). The
 * tree is executed as ONE flattened token stream whose topology is held as
 * GPU-resident segment metadata (Flide, kongchang.com page, intro and section
 * "ForkAttention: exact forking in GPU indices"). Every token attends to all
 * tokens of its ancestor segments and to the tokens of its own segment up to
 * itself; tokens of different branches never see each other (same page,
 * section "attention masks and probability distortion"). In the recurrent
 * Gated DeltaNet layer the state at the end of a parent segment is copied
 * exactly into every child (techfi24.com page, section "Exact State Forking";
 * kongchang.com page, "Gated DeltaNet layer"). Each branch's result equals an
 * isolated forward pass of that branch, up to floating-point rounding.
 *
 * Stream layout: segment s holds seg_len[s] >= 1 tokens; segments are laid out
 * contiguously in index order (segment 0 first); parent[s] is -1 for a root or
 * an index < s. T = sum(seg_len). Several roots (independent requests) may
 * share one stream.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless their name ends in _h (host).
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*); no call
 *     allocates device memory or synchronises the stream, except those marked
 *     "synchronises".
 *   - All validation happens on the host before anything is enqueued, so a
 *     call that returns an error has enqueued nothing and written nothing.
 *   - Tensors are contiguous row-major. GQA: kv head of query head h is
 *     h / (H / Hkv).
 *   - On error the call returns a negative fork_status and fork_last_error()
 *     returns a message (thread-local, valid until the next call on the same
 *     thread).
 *   - The caller owns every buffer. The library owns only fork_graph objects.
 */
#ifndef FORK_H_
#define FORK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FORK_OK = 0,
  FORK_E_ARG = -1,          /* null pointer, bad size, inconsistent arguments */
  FORK_E_TREE = -2,         /* invalid tree: parent >= s or < -1, seg_len < 1, too deep */
  FORK_E_UNSUPPORTED = -3,  /* head size or dtype with no kernel in the library */
  FORK_E_WORKSPACE = -4,    /* workspace or staging buffer too small */
  FORK_E_CAPACITY = -5,     /* tree larger than the capacities the blob was sized for */
  FORK_E_HIP = -6,          /* a HIP runtime call failed */
  FORK_E_DEVICE = -7        /* a kernel found the blob unusable (fork_meta_check) */
} fork_status;

/* Bits of the device error word of a metadata blob (fork_meta_check). Every
 * kernel that reads a blob first checks its header against the capacities
 * the launch was made for; on a mismatch the kernel sets a bit and exits
 * without reading or writing anything else, so the outputs keep their old
 * contents. fork_meta_build clears the word. */
#define FORK_DEVERR_MAGIC 1     /* the blob holds no built metadata */
#define FORK_DEVERR_CAPACITY 2  /* the blob's tree exceeds the launch's capacities (e.g. a
                                   graph recorded for one bucket replayed on a blob rebuilt
                                   with larger capacities: its workspaces would overflow) */

typedef enum { FORK_F32 = 0, FORK_BF16 = 1 } fork_dtype;

/* Capacities a metadata blob is sized for. A blob built once can hold any tree
 * within them, which is what lets a captured graph be replayed on new trees. */
typedef struct fork_caps {
  int32_t t_cap;      /* max tokens in the stream */
  int32_t s_cap;      /* max segments */
  int32_t depth_cap;  /* max segment depth (a root has depth 0) */
  int32_t gqa_group;  /* H / Hkv of the attention layers served; 1..128 */
  int32_t kv_heads;   /* Hkv of those layers, or 0. When given, query tiles with long
                         key ranges are split into parts (merged by log-sum-exp) so a
                         small tree still fills the GPU; see fork_attn_workspace. */
  int32_t ctx_cap;    /* rows of the key/value cache that cached contexts index
                         (fork_meta_build_ctx), or 0: no cached context */
} fork_caps;

/* Depths whose segment counts a fork_meta carries for launch planning. */
#define FORK_PLAN_DEPTHS 32

/* Host descriptor of a built metadata blob. The arrays live in `dev`. */
typedef struct fork_meta {
  int32_t num_tokens;      /* T */
  int32_t num_segments;    /* S */
  int32_t num_roots;       /* R */
  int32_t max_depth;       /* deepest segment depth */
  int32_t num_attn_tiles;  /* query tiles of the attention work list */
  int32_t num_chunks;      /* Gated DeltaNet chunks (never crossing a segment) */
  int32_t tile_tokens;     /* tokens per attention query tile */
  int32_t num_attn_merges; /* query tiles split into key-range parts */
  fork_caps caps;
  void* dev;               /* caller-owned device blob, >= fork_meta_size bytes */
  size_t dev_bytes;
  /* depths 0 .. min(max_depth, FORK_PLAN_DEPTHS - 1): segments at the depth,
     and those longer than one 64-token Gated DeltaNet chunk (the library uses
     them to skip kernel launches with no work outside graph capture) */
  int32_t level_segs[FORK_PLAN_DEPTHS];
  int32_t level_long[FORK_PLAN_DEPTHS];
  int32_t num_attn_parts;  /* partial-result slots (per kv head) the split query tiles use */
} fork_meta;

/* Array ids for fork_meta_export. */
enum {
  FORK_ARR_TOK_SEG = 0,      /* [T] segment of each token */
  FORK_ARR_TOK_POS = 1,      /* [T] position inside its segment */
  FORK_ARR_TOK_ISO_POS = 2,  /* [T] position in the isolated root-to-segment sequence */
  FORK_ARR_SEG_START = 3,    /* [S] first token of each segment */
  FORK_ARR_DEPTH = 4,        /* [S] number of ancestors */
  FORK_ARR_ANC_LEN = 5,      /* [S] total tokens of the ancestors */
  FORK_ARR_ROOT = 6,         /* [S] root segment of each segment */
  FORK_ARR_CTX_START = 7,    /* [S] first cache row of each root's context (0 if none) */
  FORK_ARR_CTX_LEN = 8       /* [S] cached context rows of each root (0 for non-roots) */
};

/* Bytes of device memory (dev) and of host staging a blob with these
 * capacities needs. Either output pointer may be null. */
fork_status fork_meta_size(const fork_caps* caps_h, size_t* dev_bytes_h, size_t* staging_bytes_h);

/*
 * Segment metadata builder (the GPU-resident indices of the tree).
 * Validates the tree, lays out per-segment arrays and work lists (attention
 * query tiles, Gated DeltaNet chunks and per-depth segment lists) into
 * staging_h on the host, copies them to dev with one hipMemcpyAsync on
 * `stream`, and launches a kernel that expands the per-token arrays
 * (segment, position in segment, position in the isolated sequence).
 * staging_h should be pinned host memory; it must stay untouched until the
 * stream has passed the copy. out_h receives the descriptor the forward calls
 * take.
 */
fork_status fork_meta_build(const int32_t* parent_h, const int32_t* seg_len_h,
                            int32_t num_segments, const fork_caps* caps_h,
                            void* dev, size_t dev_bytes,
                            void* staging_h, size_t staging_bytes,
                            fork_meta* out_h, void* stream);

/*
 * Host half of fork_meta_build only: validation and layout into staging_h,
 * no HIP call. Returns in *upload_bytes_h how many leading bytes of staging_h
 * fork_meta_build would copy. For tests and for callers that upload
 * themselves. out_h->dev is set to null.
 */
fork_status fork_meta_plan(const int32_t* parent_h, const int32_t* seg_len_h,
                           int32_t num_segments, const fork_caps* caps_h,
                           void* staging_h, size_t staging_bytes,
                           size_t* upload_bytes_h, fork_meta* out_h);

/*
 * Checkpoint resume: roots whose prefix was computed by an earlier pass. The
 * keys and values of that prefix stay in a caller-owned cache kc/vc
 * [ctx_cap, Hkv, D] and the stream holds only the new segments (Flide,
 * kongchang.com page, section "ForkAttention: exact forking in GPU indices":
 * growing agent histories resume from checkpoints saved by earlier passes
 * instead of being recomputed; the recurrent state of the prefix is the
 * root_state of gdn_fork_forward). For
 * root s, ctx_len_h[s] >= 0 cache rows from ctx_start_h[s] precede its first
 * token: every token of s's tree attends to them, and tok_iso_pos counts
 * them. Several roots may name the same rows (siblings resumed from one
 * shared prefix). Non-roots must have ctx_len_h 0. Ranges must lie within
 * [0, caps.ctx_cap). Both arrays null: no context (as fork_meta_build).
 * Attention over such a blob goes through fork_attn_forward_ctx.
 */
fork_status fork_meta_build_ctx(const int32_t* parent_h, const int32_t* seg_len_h,
                                const int32_t* ctx_start_h, const int32_t* ctx_len_h,
                                int32_t num_segments, const fork_caps* caps_h, void* dev,
                                size_t dev_bytes, void* staging_h, size_t staging_bytes,
                                fork_meta* out_h, void* stream);
fork_status fork_meta_plan_ctx(const int32_t* parent_h, const int32_t* seg_len_h,
                               const int32_t* ctx_start_h, const int32_t* ctx_len_h,
                               int32_t num_segments, const fork_caps* caps_h, void* staging_h,
                               size_t staging_bytes, size_t* upload_bytes_h, fork_meta* out_h);

/* Copy one metadata array (FORK_ARR_*) from the device into dst_h (int32,
 * T or S entries). Synchronises the stream. For tests. */
fork_status fork_meta_export(const fork_meta* m, int32_t array_id, int32_t* dst_h, void* stream);

/* Reads the blob's device error word (FORK_DEVERR_* bits, 0 if no kernel
 * reported a problem since the last fork_meta_build) into *device_error_h
 * (may be null). Returns FORK_E_DEVICE if the word is nonzero, FORK_OK
 * otherwise. Synchronises the stream (so every launch enqueued before it on
 * `stream` has run). Argument validation happens on the host before any
 * launch; this word covers what only the kernels can see, such as a blob
 * rewritten or rebuilt behind a recorded graph. */
fork_status fork_meta_check(const fork_meta* m, int32_t* device_error_h, void* stream);

/* Dense [T, T] uint8 visibility mask computed on the GPU from the device
 * metadata: mask[t*T + j] = 1 iff token t attends to token j. T <= 8192.
 * For tests. */
fork_status fork_meta_dense_mask(const fork_meta* m, uint8_t* mask, void* stream);

/* ---------------------------------------------------------------- attention
 * Tree-masked softmax attention over the flattened stream
 * (kongchang.com page, section "ForkAttention: exact forking in GPU indices").
 * q [T,H,D], k/v [T,Hkv,D] and o [T,H,D] of dtype dt; lse [T,H] float32 or
 * null (natural-log sum of exp of the scaled scores). Scores are scale * q.k
 * with scale <= 0 meaning 1/sqrt(D). Each prefix key/value tile is staged in
 * LDS once per query tile and reused by every packed query row (GQA heads x
 * tokens of sibling segments). Supported: D in {64, 128}; H / Hkv must equal
 * the gqa_group the metadata was built for, and Hkv its kv_heads when that is
 * nonzero. The workspace holds the partial results of split query tiles
 * (kv_heads != 0): each part's normalised output in the output dtype (so a
 * split tile's output is rounded to it once more than a whole tile's) and
 * its fp32 log-sum-exp; fork_attn_workspace gives its size for the blob's
 * capacities; it may be null when that size is 0. Work is handed out from
 * counters kept in the metadata blob (zero after fork_meta_build, reset by
 * each launch): two attention launches on one blob must not overlap in time.
 */
fork_status fork_attn_workspace(const fork_meta* m, int32_t H, int32_t Hkv, int32_t D,
                                fork_dtype dt, size_t* bytes_h);
fork_status fork_attn_forward(const fork_meta* m, const void* q, const void* k, const void* v,
                              void* o, float* lse, int32_t H, int32_t Hkv, int32_t D,
                              float scale, fork_dtype dt, void* ws, size_t ws_bytes,
                              void* stream);
/* The same with cached contexts (fork_meta_build_ctx): kc/vc [caps.ctx_cap, Hkv, D]
 * of dtype dt hold the resumed prefixes' keys and values; required (non-null)
 * when caps.ctx_cap > 0. Each context is read like a fully visible ancestor
 * range. fork_attn_forward is this call with no cache and requires
 * caps.ctx_cap == 0. */
fork_status fork_attn_forward_ctx(const fork_meta* m, const void* q, const void* k, const void* v,
                                  const void* kc, const void* vc, void* o, float* lse, int32_t H,
                                  int32_t Hkv, int32_t D, float scale, fork_dtype dt, void* ws,
                                  size_t ws_bytes, void* stream);

/* FP8 scores: fork_attn_forward with the queries and keys given as OCP FP8
 * E4M3 codes with one fp32 scale per (token, head) row (as fork_quantize_fp8
 * writes them: q8 [T, H, D] bytes with q_scale [T, H], k8 [T, Hkv, D] bytes
 * with k_scale [T, Hkv]), so that the attention scores
 *   s = scale * (q8 . k8) * q_scale[t, h] * k_scale[j, h / (H / Hkv)]
 * are formed on the FP8 matrix cores (E4M3 x E4M3, fp32 accumulation). The
 * values v [T, Hkv, D], the output o [T, H, D] and the probabilities that
 * weight the values stay bf16; lse as fork_attn_forward. Scales per row keep
 * every branch quantised exactly as in its isolated pass (a row is one
 * token). The pages report FP8 use where the hardware has it (techfi24.com
 * page, section "Exact State Forking"). Supported: D = 128, metadata without
 * cached contexts (caps.ctx_cap == 0); workspace as fork_attn_forward (bf16). */
fork_status fork_attn_forward_qk8(const fork_meta* m, const void* q8, const float* q_scale, const void* k8,
                                  const float* k_scale, const void* v, void* o, float* lse, int32_t H,
                                  int32_t Hkv, int32_t D, float scale, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fork_attn_forward_ctx without a workspace argument. The partial results of
 * split query tiles go to a scratch array compiled into the library, one
 * copy per GPU, FORK_ATTN_SCRATCH_BYTES bytes, held until the process ends.
 * The call allocates nothing. It returns FORK_E_CAPACITY when the tree's
 * split plan needs more than the array holds (num_attn_parts * Hkv slots of
 * 256 * D output-dtype values and 256 fp32 log-sum-exps each; for the
 * capacity bound of a stream being captured, every slot the blob may use).
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU race and must not be issued. Nothing in the array needs clearing:
 * each slot row the merge reads is written earlier in the same call.
 * Arguments and results are otherwise those of fork_attn_forward_ctx. */
#define FORK_ATTN_SCRATCH_BYTES ((size_t)64 << 20)
fork_status fork_attn_forward_noalloc(const fork_meta* m, const void* q, const void* k, const void* v,
                                      const void* kc, const void* vc, void* o, float* lse, int32_t H,
                                      int32_t Hkv, int32_t D, float scale, fork_dtype dt, void* stream);

/* ----------------------------------------------------------- Gated DeltaNet
 * Forked Gated DeltaNet: per head, the dv x dk state follows
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = scale * S_t q_t
 * along each branch; a segment starts from its parent's end state (the fork:
 * that state is written exactly into seg_start_state of every child), a root
 * from root_state or zero. (The pages describe the layer and the fork in
 * prose: techfi24.com page, "Exact State Forking"; kongchang.com page,
 * "Gated DeltaNet layer".)
 * q/k [T,H,dk], v [T,H,dv], o [T,H,dv] of dtype dt; a/b [T,H] float32,
 * the decay gate a in [0, 1] (a = 0 forgets the state at that token; the
 * chunked kernels floor log a at -20, so a gate below e^-20 acts as e^-20,
 * which moves no decay factor by more than 2.1e-9);
 * root_state [R,H,dv,dk] float32 or null (zero; R roots in index order);
 * seg_start_state [S,H,dv,dk] float32 (required: the fork copies);
 * seg_final_state [S,H,dv,dk] float32 or null. States are row-major dv x dk.
 * Supported: dk == dv in {32, 64, 128}. The workspace holds per-chunk
 * intermediates; gdn_fork_workspace sizes it for the blob's capacities.
 * With seg_final_state null (bf16, dk == 128), runs of consecutive leaf
 * siblings of at most 64 tokens in total are computed together in one chunk
 * from their shared start state (their outputs agree with the one-by-one
 * computation to rounding; every start state, and so every fork copy, is
 * bit for bit the same). Work is handed out from counters in the metadata
 * blob, reset by each launch: two launches on one blob must not overlap.
 */
fork_status gdn_fork_workspace(const fork_meta* m, int32_t H, int32_t dk, int32_t dv,
                               fork_dtype dt, size_t* bytes_h);
fork_status gdn_fork_forward(const fork_meta* m, const void* q, const void* k, const void* v,
                             const float* a, const float* b, const float* root_state,
                             void* o, float* seg_start_state, float* seg_final_state,
                             int32_t H, int32_t dk, int32_t dv, float scale, fork_dtype dt,
                             void* ws, size_t ws_bytes, void* stream);

/* FP8 inputs: gdn_fork_forward with q, k and v given as OCP FP8 E4M3 codes
 * with one fp32 scale per (token, head) row, as fork_quantize_fp8 writes
 * them: q8, k8, v8 [T, H, 128] bytes (16-byte aligned) with q_scale, k_scale,
 * v_scale [T, H]; the row's values are code * scale. Scales must be positive
 * normal floats (the quantiser's max|row| / 448, or 1 for a zero row). The
 * kernel reads the codes (half the bytes of bf16 inputs) and decodes them on
 * chip exactly; the per-row scales enter as fp32 factors of b, of the value
 * rows and of the output rows (the recurrence is the same recurrence in the
 * codes, see gdn.hip), so the state matches the bf16 recurrence on the
 * decoded values to rounding. The pages' Gated DeltaNet kernel uses FP8
 * where the hardware has it (techfi24.com page, section "Exact State
 * Forking"). o [T, H, 128] bf16; a, b, root_state, seg_start_state and
 * seg_final_state as gdn_fork_forward (leaf siblings packed when
 * seg_final_state is null). Supported: dk = dv = 128. Every segment runs on
 * the per-(segment, head) fused kernel, so no workspace is needed. Work
 * counters as gdn_fork_forward: launches on one blob must not overlap. */
fork_status gdn_fork_forward_fp8(const fork_meta* m, const void* q8, const float* q_scale, const void* k8,
                                 const float* k_scale, const void* v8, const float* v_scale, const float* a,
                                 const float* b, const float* root_state, void* o, float* seg_start_state,
                                 float* seg_final_state, int32_t H, int32_t dk, int32_t dv, float scale,
                                 void* stream);

/* ------------------------------------------------------------ block pieces
 * Fork-aware operations around the two layers of a hybrid block. Each branch
 * must evaluate exactly as its isolated forward pass (kongchang.com page,
 * section "ForkAttention: exact forking in GPU indices"), so an operation that
 * reads a token's position or its predecessors reads them in the token's
 * isolated sequence, from the same metadata. Both calls read T from the blob
 * (capture-safe) and touch rows < T only.
 */

/* Rotary position embedding, in place, at each token's isolated position
 * (tok_iso_pos: its root's resumed context, its ancestors' tokens, then its
 * own position). x [T, nheads, D] of dtype dt; for i < D/2 the pair
 * (x_i, x_{i+D/2}) of each head rotates by the angle tok_iso_pos * theta^(-2i/D).
 * D a multiple of 8 in 8..256; theta > 1. */
fork_status fork_rope_forward(const fork_meta* m, void* x, int32_t nheads, int32_t D, float theta,
                              fork_dtype dt, void* stream);

/* The same rotation out of place from a strided source: head h of token t is
 * read at src[t * ld_src + h * D ...] and written to dst [T, nheads, D]
 * (contiguous). theta 0 copies without rotating. This splits the output of a
 * fused projection ([T, ld_src], several tensors side by side) into
 * contiguous heads, rotating q and k on the way. ld_src >= nheads * D and a
 * multiple of 4; src and dst aligned to 4 elements and not overlapping (over
 * caps.t_cap rows). */
fork_status fork_rope_copy_forward(const fork_meta* m, const void* src, int64_t ld_src, void* dst, int32_t nheads,
                                   int32_t D, float theta, fork_dtype dt, void* stream);

/* Causal depthwise convolution of width K (2..8) along each token's isolated
 * sequence (the short convolution in front of a Gated DeltaNet layer):
 *   y[t][c] = act(bias[c] + sum_{j<K} w[c*K + K-1-j] * in_c(t, j)),
 * in_c(t, j) channel c of the input j tokens before t in its isolated
 * sequence: within t's segment, then the parent's last tokens (and further
 * ancestors when a parent is shorter than the window); before a root's first
 * token, conv_state[r][c][K-1-j'] for the j'-th input before it (the saved
 * last K-1 inputs of a resumed context, oldest first; r the root's ordinal
 * among roots), or zero when conv_state is null. x, y [T, C] of dtype dt, not
 * overlapping, C a multiple of 8; w [C, K] (16-byte aligned), bias [C] (or
 * null) and conv_state [R, C, K-1] (or null) fp32. act: 0 identity, 1 SiLU. */
fork_status fork_conv_forward(const fork_meta* m, const void* x, const float* w, const float* bias,
                              const float* conv_state, void* y, int32_t C, int32_t K, int32_t act,
                              fork_dtype dt, void* stream);

/* ------------------------------------------------------------ mixer pieces
 * Per-token operations of the two token mixers of a hybrid block. They read
 * no other token, so on the flattened stream every branch gets exactly its
 * isolated result and the shared prefix is processed once (kongchang.com
 * page, section "ForkAttention: exact forking in GPU indices"). The pages do
 * not spell out the block around the layers; these forms follow the published
 * Gated DeltaNet layer (short convolution + SiLU, L2-normalised query and
 * key, softplus decay, sigmoid write strength, gated RMS norm at the output)
 * and a sigmoid output gate on attention. */

/* Gate / norm over rows of D elements, T * nheads rows (T from the blob):
 *   mode 0: y = x * sigmoid(g)
 *   mode 1: y = x / sqrt(mean(x^2) + eps) * w * silu(g),  silu(g) = g sigmoid(g)
 *   mode 2: y = x / sqrt(mean(x^2) + eps) * w             (g unused, may be null)
 * x, y [T, nheads, D] of dtype dt (y may be x); g of dtype dt with token t's
 * heads at g + t * ld_g (ld_g = 0 means nheads * D, i.e. g [T, nheads, D];
 * otherwise >= nheads * D and a multiple of 8, so g can be a column block of
 * a wider projection output), 16-byte aligned; w [D] fp32, 16-byte aligned,
 * the same for every head (modes 1, 2). D a multiple of 8 in 8..65536;
 * eps > 0 for modes 1, 2. */
fork_status fork_gate_forward(const fork_meta* m, const void* x, const void* g, int64_t ld_g, const float* w,
                              void* y, int32_t nheads, int32_t D, int32_t mode, float eps, fork_dtype dt,
                              void* stream);

/* Gated DeltaNet inputs after the short convolution, per token t and head h:
 *   q[t,h] = c_q / sqrt(|c_q|^2 + eps),  k[t,h] = c_k / sqrt(|c_k|^2 + eps),
 *   v[t,h] = c_v,
 *   a[t,h] = exp(-exp(a_log[h]) * softplus(ab[t,h] + dt_bias[h])),
 *   b[t,h] = sigmoid(ab[t,H+h]),
 * with c [T, 2 H dk + H dv] holding the query heads, then the key heads, then
 * the value heads of each token, and ab the decay and write-strength
 * projections (2 H values of token t at ab + t * ld_ab; ld_ab = 0 means 2 H,
 * otherwise >= 2 H), both of dtype dt; q, k [T,H,dk], v [T,H,dv] of dtype dt, and
 * a, b [T,H] fp32: the inputs of gdn_fork_forward. a_log, dt_bias [H] fp32.
 * c may be null: then only a and b are formed (q, k, v ignored; see
 * gdn_conv_inputs_forward). dk, dv multiples of 8 in 8..1024; eps > 0. T
 * from the blob. */
fork_status gdn_inputs_forward(const fork_meta* m, const void* c, const void* ab, int64_t ld_ab, const float* a_log,
                               const float* dt_bias, void* q, void* k, void* v, float* a, float* b, int32_t H,
                               int32_t dk, int32_t dv, float eps, fork_dtype dt, void* stream);

/* The short convolution of the Gated DeltaNet projections and their split in
 * one pass: fork_conv_forward with SiLU over x [T, 2 H dk + H dv] (query
 * heads, key heads, value heads of each token; same taps, bias and
 * conv_state conventions, C = 2 H dk + H dv), then the query and key heads
 * L2-normalised, u / sqrt(|u|^2 + eps), and the three parts written to
 * q, k [T,H,dk] and v [T,H,dv] (dtype dt), as gdn_inputs_forward would
 * produce from the convolution's output. dk == dv, a power of two in
 * 8..512; K 2..8; w 16-byte aligned. */
fork_status gdn_conv_inputs_forward(const fork_meta* m, const void* x, const float* w, const float* bias,
                                    const float* conv_state, void* q, void* k, void* v, int32_t H, int32_t dk,
                                    int32_t dv, int32_t K, float eps, fork_dtype dt, void* stream);

/* Projection y [M, N] = x [M, K] w [N, K]^T, or with accumulate = 1
 * y += x w^T (a residual connection folded into the product), all row-major
 * of dtype dt, fp32 accumulation (hipBLASLt). Rows are tokens of the
 * flattened stream: one call projects every branch, the shared prefix once.
 * y must not overlap x or w.
 * The first call on a device creates a hipBLASLt handle and a 32 MiB
 * workspace, kept for the process. The first call per (M, N, K, dt) times
 * the heuristic's candidate algorithms once on its operands (into a scratch
 * output it allocates and frees; it synchronises the stream) and keeps the
 * fastest, so make that first call outside any graph capture. Calls are
 * serialised by a lock. */
fork_status fork_linear_forward(const void* x, const void* w, void* y, int32_t M, int32_t N, int32_t K,
                                int32_t accumulate, fork_dtype dt, void* stream);

/* ------------------------------------------------------------------ FP8
 * FP8 execution where the hardware has it (techfi24.com page, "Exact State
 * Forking" section: the kernels use FP8 when available and a large model is
 * run quantised to FP8). Format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals, largest finite 448, no
 * infinities), one byte per value, with one fp32 scale per row:
 * value = decode(code) * scale[row]. A row of activations is one token, so a
 * token's codes depend on that token alone and every branch of the stream is
 * quantised exactly as in its isolated pass. */

/* Row-wise quantisation of x [rows, K] (dtype dt) to codes q [rows, K] (bytes):
 *   scales[r] = max_k |x[r][k]| / 448 (1 for an all-zero row),
 *   q[r][k]   = E4M3 nearest-even rounding of clamp(x[r][k] / scales[r], -448, 448),
 * both divisions correctly rounded fp32. scales [rows] fp32 (device). K a
 * positive multiple of 8; x 16-byte and q 8-byte aligned. */
fork_status fork_quantize_fp8(const void* x, void* q, float* scales, int64_t rows, int32_t K, fork_dtype dt,
                              void* stream);

/* FP8 projection y [M, N] (bf16) with
 *   y[m][n] = (sum_k xq[m][k] wq[n][k]) * x_scale[m] * w_scale[n]
 * (or y += that with accumulate = 1): E4M3 codes with row scales as written
 * by fork_quantize_fp8 (x_scale [M], w_scale [N], device), fp32 accumulation
 * on the FP8 matrix cores (hipBLASLt). K a multiple of 16. Handle, workspace
 * and algorithm choice as fork_linear_forward. */
fork_status fork_linear_fp8_forward(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                                    void* y, int32_t M, int32_t N, int32_t K, int32_t accumulate, void* stream);

/* ---------------------------------------------------------- decision readout
 * Per-option probabilities of a decision request: the pages measure the
 * engine by the probabilities it gives each candidate option, as their total
 * variation distance to a float32 reference (kongchang.com page, section on
 * performance) and by whether the chosen option stays the same (openai-hub.com
 * page, section on the six variables); they define no scoring head. Reading
 * taken: the options are the leaf segments; leaves sharing a parent form one
 * decision group; for every option c
 *   score[c] = sum_i w[i] * x[last token of c, i] / sqrt(C),
 *   prob[c]  = exp(score[c]) / sum over c' in c's group of exp(score[c']),
 * with fp32 accumulation (the softmax shifted by the group's maximum). Every
 * segment that is not an option (roots, segments with children) gets score 0
 * and prob 0. x [T, C] of dtype dt (a layer's output rows, e.g. o [T, H, D]
 * with C = H * D), w [C] fp32, score and prob [S] fp32 (device, S from the
 * blob); x and w 16-byte aligned, C a multiple of 8 in 8..65536. Two kernel
 * launches, no allocation, no synchronisation, deterministic. */
fork_status fork_option_readout(const fork_meta* m, const void* x, const float* w, int32_t C, float* score,
                                float* prob, fork_dtype dt, void* stream);

/* ------------------------------------------------------------ graph buckets
 * A compact set of pre-recorded execution graphs serves varied request mixes
 * (kongchang.com page, section "pre-recorded execution graphs"). A fork_graph
 * records fork_attn_forward followed by gdn_fork_forward for a metadata blob
 * with fixed capacities (the bucket); its kernels read the tree from the blob
 * at run time. To run a new tree: fork_meta_build into the same blob (same
 * capacities, same dev pointer), then fork_graph_launch. All buffers in args
 * must be sized for the bucket's t_cap / s_cap and stay valid while the graph
 * lives. Tokens beyond the current T are neither read nor written.
 */
typedef struct fork_graph_args {
  /* attention */
  const void *q, *k, *v;
  void* o;
  float* lse;
  int32_t H, Hkv, D;
  float scale;
  void* attn_ws;
  size_t attn_ws_bytes;
  /* Gated DeltaNet */
  const void *gq, *gk, *gv;
  const float *a, *b, *root_state;
  void* go;
  float *seg_start_state, *seg_final_state;
  int32_t gH, dk, dv;
  float gscale;
  void* gdn_ws;
  size_t gdn_ws_bytes;
  fork_dtype dt;
  /* key/value cache of resumed contexts, [caps.ctx_cap, Hkv, D]; required when
     caps.ctx_cap > 0, else null */
  const void *kc, *vc;
} fork_graph_args;

typedef struct fork_graph fork_graph;

fork_status fork_graph_create(const fork_meta* m, const fork_graph_args* args_h, void* stream,
                              fork_graph** out_h);
fork_status fork_graph_launch(fork_graph* g, void* stream);
fork_status fork_graph_destroy(fork_graph* g);

/* Message for the last error on this thread ("" if none). */
const char* fork_last_error(void);

/* Library version string. */
const char* fork_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FORK_H_ */
