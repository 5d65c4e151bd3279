/*
 * CPU oracle for tree-flattened ForkAttention and the forked Gated DeltaNet.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path never
 * calls it and shares no code, header, table or helper with it.
 *
 * Built twice from this one file: with REAL=double (the parity reference) and
 * with REAL=float (the float32 reference that total-variation distance is
 * quoted against on the Flide pages, kongchang.com page, section
 * "Performance": engines are ranked by their distance to a float32 reference).
 *
 * What is computed (plain and slow on purpose):
 *   A decision request is a tree of segments flattened into one token stream
 *   (kongchang.com page, intro and section "ForkAttention: exact forking in GPU
 *   indices"). The result for every branch must equal an isolated forward pass
 *   of that branch. So for every segment s this file builds the isolated
 *   sequence X_s = the token ranges of s's ancestors, root first, then s
 *   itself, and runs each layer over X_s as an ordinary sequence, keeping only
 *   the rows of s. Nothing is shared between segments.
 *
 *   - Softmax attention: causal attention over X_s (every token of an ancestor
 *     is earlier than every token of s), GQA with contiguous head groups
 *     (kv head = h / (H / Hkv)).
 *   - Gated DeltaNet: the token recurrence
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = scale * S_t q_t
 *     run from the root's saved state (or zero) over X_s in order. The state
 *     just before s's first token is s's start state (the exact fork copy of
 *     the parent's end state), the state after its last token its final state.
 *
 * Parity status: every function here is pinned by tests that do not reuse this
 * code (brute force over the flattened stream with a dense tree mask, library
 * scaled-dot-product attention on single-segment trees, closed forms of the
 * recurrence, and an independent index computation for the metadata).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef REAL
#define REAL double
#endif

#define ORACLE_OK 0
#define ORACLE_E_TREE (-2)
#define ORACLE_E_ARG (-1)

#define ORACLE_MAX_PATH 512

/* Tree checks: parent[s] == -1 or 0 <= parent[s] < s; seg_len[s] >= 1; a
 * root-to-segment path holds at most ORACLE_MAX_PATH segments. */
static int check_tree(int S, const int32_t* parent, const int32_t* seg_len) {
  if (S <= 0 || !parent || !seg_len) return ORACLE_E_ARG;
  int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * S);
  int bad = 0;
  for (int s = 0; s < S && !bad; ++s) {
    if (seg_len[s] < 1 || parent[s] < -1 || parent[s] >= s) bad = 1;
    else depth[s] = parent[s] < 0 ? 0 : depth[parent[s]] + 1;
    if (!bad && depth[s] >= ORACLE_MAX_PATH) bad = 1;
  }
  free(depth);
  return bad ? ORACLE_E_TREE : ORACLE_OK;
}

static long long total_tokens(int S, const int32_t* seg_len) {
  long long T = 0;
  for (int s = 0; s < S; ++s) T += seg_len[s];
  return T;
}

/* Path of s: ancestors root first, then s. Returns its length. */
static int build_path(int s, const int32_t* parent, int32_t* path, int cap) {
  int n = 0;
  for (int x = s; x >= 0; x = parent[x]) {
    if (n >= cap) return -1;
    path[n++] = x;
  }
  for (int i = 0; i < n / 2; ++i) {
    int32_t t = path[i];
    path[i] = path[n - 1 - i];
    path[n - 1 - i] = t;
  }
  return n;
}

int oracle_num_tokens(int S, const int32_t* parent, const int32_t* seg_len, long long* T) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  *T = total_tokens(S, seg_len);
  return ORACLE_OK;
}

/*
 * Segment and token metadata, straight from the definitions:
 *   seg_start[s] = sum of seg_len[r] for r < s (segments laid out in index order)
 *   depth[s]     = number of ancestors; root[s] = the root of s's tree
 *   anc_len[s]   = total tokens of s's ancestors
 *   tok_seg[t]   = the segment holding token t; tok_pos[t] = t - seg_start[seg]
 *   tok_iso_pos[t] = anc_len[seg] + tok_pos[t], the token's position in the
 *                    isolated sequence of its segment.
 */
/* Resumed contexts (kongchang.com page, section "ForkAttention: exact forking
 * in GPU indices": agent histories resume from checkpoints of earlier passes).
 * ctx_len[s] (nullable) cached tokens precede root s; non-roots have none. */
static int check_ctx(int S, const int32_t* parent, const int32_t* ctx_start, const int32_t* ctx_len) {
  if ((ctx_start == NULL) != (ctx_len == NULL)) return ORACLE_E_ARG;
  if (!ctx_len) return ORACLE_OK;
  for (int s = 0; s < S; ++s)
    if (ctx_len[s] < 0 || (ctx_len[s] > 0 && (parent[s] >= 0 || ctx_start[s] < 0))) return ORACLE_E_ARG;
  return ORACLE_OK;
}

/* As oracle_meta, with the positions counting the root's resumed context:
 * tok_iso_pos[t] = ctx_len[root] + anc_len[seg] + tok_pos[t]. */
int oracle_meta_ctx(int S, const int32_t* parent, const int32_t* seg_len, const int32_t* ctx_len,
                    int32_t* seg_start, int32_t* depth, int32_t* root, int32_t* anc_len,
                    int32_t* tok_seg, int32_t* tok_pos, int32_t* tok_iso_pos);

int oracle_meta(int S, const int32_t* parent, const int32_t* seg_len,
                int32_t* seg_start, int32_t* depth, int32_t* root, int32_t* anc_len,
                int32_t* tok_seg, int32_t* tok_pos, int32_t* tok_iso_pos) {
  return oracle_meta_ctx(S, parent, seg_len, NULL, seg_start, depth, root, anc_len, tok_seg, tok_pos,
                         tok_iso_pos);
}

int oracle_meta_ctx(int S, const int32_t* parent, const int32_t* seg_len, const int32_t* ctx_len,
                    int32_t* seg_start, int32_t* depth, int32_t* root, int32_t* anc_len,
                    int32_t* tok_seg, int32_t* tok_pos, int32_t* tok_iso_pos) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  if (ctx_len)
    for (int s = 0; s < S; ++s)
      if (ctx_len[s] < 0 || (ctx_len[s] > 0 && parent[s] >= 0)) return ORACLE_E_ARG;
  int32_t acc = 0;
  for (int s = 0; s < S; ++s) {
    seg_start[s] = acc;
    acc += seg_len[s];
  }
  for (int s = 0; s < S; ++s) {
    int d = 0, r = s;
    int32_t al = 0;
    for (int x = parent[s]; x >= 0; x = parent[x]) {
      ++d;
      al += seg_len[x];
      r = x;
    }
    depth[s] = d;
    root[s] = r;
    anc_len[s] = al;
  }
  for (int s = 0; s < S; ++s)
    for (int i = 0; i < seg_len[s]; ++i) {
      int32_t t = seg_start[s] + i;
      tok_seg[t] = s;
      tok_pos[t] = i;
      tok_iso_pos[t] = (ctx_len ? ctx_len[root[s]] : 0) + anc_len[s] + i;
    }
  return ORACLE_OK;
}

/*
 * Dense visibility mask over the flattened stream, mask[t*T + j] = 1 iff token
 * t may attend to token j: j belongs to an ancestor segment of t's segment, or
 * to t's own segment at a position not after t. Tokens of different branches
 * never see each other (kongchang.com page, section "attention masks and
 * probability distortion").
 */
int oracle_mask(int S, const int32_t* parent, const int32_t* seg_len, uint8_t* mask) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  long long T = total_tokens(S, seg_len);
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t acc = 0;
  for (int s = 0; s < S; ++s) { start[s] = acc; acc += seg_len[s]; }
  memset(mask, 0, (size_t)(T * T));
  for (int s = 0; s < S; ++s) {
    for (int i = 0; i < seg_len[s]; ++i) {
      long long t = start[s] + i;
      uint8_t* row = mask + t * T;
      for (int x = parent[s]; x >= 0; x = parent[x])
        for (int j = 0; j < seg_len[x]; ++j) row[start[x] + j] = 1;
      for (int j = 0; j <= i; ++j) row[start[s] + j] = 1;
    }
  }
  free(start);
  return ORACLE_OK;
}

/*
 * Tree attention, one isolated sequence per segment.
 * q [T,H,D], k/v [T,Hkv,D] (float32 stream layout). For every selected segment
 * s, head h, own token at isolated position n: z_j = scale * q.k_j over the
 * first n+1 tokens of X_s, m = max z, l = sum_j exp(z_j - m) in j order,
 * o = sum_j exp(z_j - m) v_j / l, lse = m + log l.
 * With resumed contexts (ctx_start/ctx_len non-null, kc/vc [*, Hkv, D] float32),
 * X_s begins with the context of s's root: cache rows ctx_start[r] ..
 * ctx_start[r] + ctx_len[r] - 1 of kc/vc, before the ancestors' tokens.
 * tok_select (nullable, [T]): compute only the rows of tokens with a nonzero
 * flag. o [T,H,D], lse [T,H] (nullable). Rows not computed are left untouched.
 */
int oracle_attention_ctx(int S, const int32_t* parent, const int32_t* seg_len,
                         const int32_t* ctx_start, const int32_t* ctx_len,
                         int H, int Hkv, int D, double scale,
                         const float* q, const float* k, const float* v,
                         const float* kc, const float* vc,
                         const uint8_t* tok_select, REAL* o, REAL* lse);

int oracle_attention(int S, const int32_t* parent, const int32_t* seg_len,
                     int H, int Hkv, int D, double scale,
                     const float* q, const float* k, const float* v,
                     const uint8_t* tok_select, REAL* o, REAL* lse) {
  return oracle_attention_ctx(S, parent, seg_len, NULL, NULL, H, Hkv, D, scale, q, k, v, NULL, NULL,
                              tok_select, o, lse);
}

int oracle_attention_ctx(int S, const int32_t* parent, const int32_t* seg_len,
                         const int32_t* ctx_start, const int32_t* ctx_len,
                         int H, int Hkv, int D, double scale,
                         const float* q, const float* k, const float* v,
                         const float* kc, const float* vc,
                         const uint8_t* tok_select, REAL* o, REAL* lse) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  if (H <= 0 || Hkv <= 0 || D <= 0 || H % Hkv != 0 || !q || !k || !v || !o) return ORACLE_E_ARG;
  e = check_ctx(S, parent, ctx_start, ctx_len);
  if (e) return e;
  if (ctx_len && (!kc || !vc)) return ORACLE_E_ARG;
  const int G = H / Hkv;
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t acc = 0;
  for (int s = 0; s < S; ++s) { start[s] = acc; acc += seg_len[s]; }

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      if (tok_select) {
        int any = 0;
        for (int j = 0; j < seg_len[s] && !any; ++j) any = tok_select[start[s] + j] != 0;
        if (!any) continue;
      }
      const int g = h / G;
      int32_t path[ORACLE_MAX_PATH];
      int np = build_path(s, parent, path, ORACLE_MAX_PATH);
      /* X_s in order: the root's context rows (cache row c as -1 - c), then
         the stream token ids of the path's segments */
      const int r = path[0];
      const int nc = ctx_len ? ctx_len[r] : 0;
      long long N = nc;
      for (int i = 0; i < np; ++i) N += seg_len[path[i]];
      int32_t* X = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
      long long n = 0;
      for (int j = 0; j < nc; ++j) X[n++] = -1 - (ctx_start[r] + j);
      for (int i = 0; i < np; ++i)
        for (int j = 0; j < seg_len[path[i]]; ++j) X[n++] = start[path[i]] + j;
      REAL* z = (REAL*)malloc(sizeof(REAL) * (size_t)N);
      const long long own0 = N - seg_len[s];
      for (long long pos = own0; pos < N; ++pos) {
        const long long t = X[pos];
        if (tok_select && !tok_select[t]) continue;
        const float* qt = q + (t * H + h) * D;
        REAL m = -INFINITY;
        for (long long j = 0; j <= pos; ++j) {
          const float* kj = X[j] >= 0 ? k + ((long long)X[j] * Hkv + g) * D
                                      : kc + ((long long)(-1 - X[j]) * Hkv + g) * D;
          REAL dot = 0;
          for (int d = 0; d < D; ++d) dot += (REAL)qt[d] * (REAL)kj[d];
          z[j] = (REAL)scale * dot;
          if (z[j] > m) m = z[j];
        }
        REAL l = 0;
        for (long long j = 0; j <= pos; ++j) {
          z[j] = exp(z[j] - m);
          l += z[j];
        }
        REAL* ot = o + (t * H + h) * D;
        for (int d = 0; d < D; ++d) {
          REAL sacc = 0;
          for (long long j = 0; j <= pos; ++j)
            sacc += z[j] * (REAL)(X[j] >= 0 ? v[((long long)X[j] * Hkv + g) * D + d]
                                            : vc[((long long)(-1 - X[j]) * Hkv + g) * D + d]);
          ot[d] = sacc / l;
        }
        if (lse) lse[t * H + h] = m + log(l);
      }
      free(z);
      free(X);
    }
  }
  free(start);
  return ORACLE_OK;
}

/*
 * Forked Gated DeltaNet, one isolated sequence per segment, recurrent form.
 * q/k [T,H,dk], v [T,H,dv], a/b [T,H] float32; root_state [R,H,dv,dk] (R =
 * number of roots, in index order) or NULL for zero. The state S is dv x dk,
 * row-major. For every token tau of X_s in order:
 *     u = S k_tau                       (dv)
 *     S = a_tau S + b_tau (v_tau - a_tau u) k_tau^T
 *     o_tau = scale * S q_tau           (kept for own tokens only)
 * which is S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T expanded.
 * seg_start_state/seg_final_state [S,H,dv,dk] (nullable) receive the state
 * before s's first token and after its last.
 */
int oracle_gdn(int S, const int32_t* parent, const int32_t* seg_len,
               int H, int dk, int dv, double scale,
               const float* q, const float* k, const float* v,
               const float* a, const float* b, const float* root_state,
               const uint8_t* seg_select, REAL* o,
               REAL* seg_start_state, REAL* seg_final_state) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  if (H <= 0 || dk <= 0 || dv <= 0 || !q || !k || !v || !a || !b || !o) return ORACLE_E_ARG;
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t* root_ord = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t acc = 0, nroot = 0;
  for (int s = 0; s < S; ++s) {
    start[s] = acc;
    acc += seg_len[s];
    root_ord[s] = parent[s] < 0 ? nroot++ : -1;
  }
  const size_t SZ = (size_t)dv * dk;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    for (int h = 0; h < H; ++h) {
      if (seg_select && !seg_select[s]) continue;
      int32_t path[ORACLE_MAX_PATH];
      int np = build_path(s, parent, path, ORACLE_MAX_PATH);
      REAL* St = (REAL*)malloc(sizeof(REAL) * SZ);
      REAL* u = (REAL*)malloc(sizeof(REAL) * dv);
      const int r = root_ord[path[0]];
      for (size_t i = 0; i < SZ; ++i)
        St[i] = root_state ? (REAL)root_state[((size_t)r * H + h) * SZ + i] : (REAL)0;
      for (int pi = 0; pi < np; ++pi) {
        const int x = path[pi];
        const int own = (x == s);
        if (own && seg_start_state) {
          REAL* dst = seg_start_state + ((size_t)s * H + h) * SZ;
          for (size_t i = 0; i < SZ; ++i) dst[i] = St[i];
        }
        for (int j = 0; j < seg_len[x]; ++j) {
          const long long t = start[x] + j;
          const float* kt = k + (t * H + h) * dk;
          const float* vt = v + (t * H + h) * dv;
          const float* qt = q + (t * H + h) * dk;
          const REAL at = a[t * H + h], bt = b[t * H + h];
          for (int r2 = 0; r2 < dv; ++r2) {
            REAL sacc = 0;
            for (int c = 0; c < dk; ++c) sacc += St[(size_t)r2 * dk + c] * (REAL)kt[c];
            u[r2] = sacc;
          }
          for (int r2 = 0; r2 < dv; ++r2) {
            const REAL w = bt * ((REAL)vt[r2] - at * u[r2]);
            for (int c = 0; c < dk; ++c)
              St[(size_t)r2 * dk + c] = at * St[(size_t)r2 * dk + c] + w * (REAL)kt[c];
          }
          if (own) {
            REAL* ot = o + (t * H + h) * dv;
            for (int r2 = 0; r2 < dv; ++r2) {
              REAL sacc = 0;
              for (int c = 0; c < dk; ++c) sacc += St[(size_t)r2 * dk + c] * (REAL)qt[c];
              ot[r2] = (REAL)scale * sacc;
            }
          }
        }
        if (own && seg_final_state) {
          REAL* dst = seg_final_state + ((size_t)s * H + h) * SZ;
          for (size_t i = 0; i < SZ; ++i) dst[i] = St[i];
        }
      }
      free(u);
      free(St);
    }
  }
  free(root_ord);
  free(start);
  return ORACLE_OK;
}

/*
 * Fork-aware pieces of a hybrid block around the two layers. Each branch must
 * evaluate exactly as an isolated forward pass (kongchang.com page, section
 * "ForkAttention: exact forking in GPU indices"), so anything that reads a
 * token's position or its predecessors reads them in the isolated sequence:
 *
 * Rotary position embedding at the isolated position n of token t (its
 * root's resumed context, ancestors and own predecessors counted): for each
 * head and i < D/2 the pair (x_i, x_{i+D/2}) rotates by the angle
 * n * theta^(-2i/D):
 *   y_i = x_i cos(a) - x_{i+D/2} sin(a),  y_{i+D/2} = x_{i+D/2} cos(a) + x_i sin(a).
 * x [T,nh,D] float32 stream layout, y [T,nh,D]; ctx_len nullable.
 */
int oracle_rope(int S, const int32_t* parent, const int32_t* seg_len, const int32_t* ctx_len,
                int nh, int D, double theta, const float* x, REAL* y) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  if (nh <= 0 || D <= 0 || D % 2 || !x || !y) return ORACLE_E_ARG;
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t acc = 0;
  for (int s = 0; s < S; ++s) { start[s] = acc; acc += seg_len[s]; }
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    int32_t path[ORACLE_MAX_PATH];
    const int np = build_path(s, parent, path, ORACLE_MAX_PATH);
    long long n0 = ctx_len ? ctx_len[path[0]] : 0;  /* isolated position of s's first token */
    for (int i = 0; i + 1 < np; ++i) n0 += seg_len[path[i]];
    for (int j = 0; j < seg_len[s]; ++j) {
      const long long t = start[s] + j;
      const REAL n = (REAL)(n0 + j);
      for (int h = 0; h < nh; ++h) {
        const float* xt = x + (t * nh + h) * D;
        REAL* yt = y + (t * nh + h) * D;
        for (int i = 0; i < D / 2; ++i) {
          const REAL ang = n * pow((REAL)theta, -2.0 * i / D);
          const REAL c = cos(ang), sn = sin(ang);
          yt[i] = (REAL)xt[i] * c - (REAL)xt[i + D / 2] * sn;
          yt[i + D / 2] = (REAL)xt[i + D / 2] * c + (REAL)xt[i] * sn;
        }
      }
    }
  }
  free(start);
  return ORACLE_OK;
}

/*
 * Causal depthwise convolution along the isolated sequence (the short
 * convolution a Gated DeltaNet block applies to its q, k, v before the
 * recurrence; not on the pages, it follows from the isolated-pass rule): for
 * channel c and the token at isolated position n,
 *   u = bias[c] + sum_{j=0}^{K-1} w[c*K + K-1-j] * in(n - j),
 * in(m) the channel's input at isolated position m: the token there for
 * m >= 0, else (m >= -(K-1)) conv_state[r][c][K-1+m] of the sequence's root
 * (the last K-1 inputs of its resumed context, oldest first) when given,
 * else 0. act 1: y = u * sigmoid(u) (SiLU); act 0: y = u.
 * x [T,C] float32, w [C,K], bias [C] (nullable), conv_state [R,C,K-1] (nullable,
 * roots in index order), y [T,C].
 */
int oracle_conv(int S, const int32_t* parent, const int32_t* seg_len, int C, int K, int act,
                const float* x, const float* w, const float* bias, const float* conv_state, REAL* y) {
  int e = check_tree(S, parent, seg_len);
  if (e) return e;
  if (C <= 0 || K <= 0 || act < 0 || act > 1 || !x || !w || !y) return ORACLE_E_ARG;
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t* root_ord = (int32_t*)malloc(sizeof(int32_t) * S);
  int32_t acc = 0, R = 0;
  for (int s = 0; s < S; ++s) {
    start[s] = acc;
    acc += seg_len[s];
    root_ord[s] = parent[s] < 0 ? R++ : -1;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < S; ++s) {
    int32_t path[ORACLE_MAX_PATH];
    const int np = build_path(s, parent, path, ORACLE_MAX_PATH);
    long long N = 0;
    for (int i = 0; i < np; ++i) N += seg_len[path[i]];
    int32_t* X = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
    long long n = 0;
    for (int i = 0; i < np; ++i)
      for (int j = 0; j < seg_len[path[i]]; ++j) X[n++] = start[path[i]] + j;
    const int r = root_ord[path[0]];
    for (long long pos = N - seg_len[s]; pos < N; ++pos) {
      const long long t = X[pos];
      for (int c = 0; c < C; ++c) {
        REAL u = bias ? (REAL)bias[c] : (REAL)0;
        for (int j = 0; j < K; ++j) {
          const long long m = pos - j;
          REAL in = 0;
          if (m >= 0) in = (REAL)x[(long long)X[m] * C + c];
          else if (conv_state && m >= -(K - 1)) in = (REAL)conv_state[((long long)r * C + c) * (K - 1) + (K - 1) + m];
          u += (REAL)w[c * K + K - 1 - j] * in;
        }
        y[t * C + c] = act ? u / (1 + exp(-u)) : u;
      }
    }
    free(X);
  }
  free(root_ord);
  free(start);
  return ORACLE_OK;
}

int oracle_real_bytes(void) { return (int)sizeof(REAL); }

#ifdef _OPENMP
#include <omp.h>
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int oracle_max_threads(void) { return omp_get_max_threads(); }
#else
void oracle_set_threads(int n) { (void)n; }
int oracle_max_threads(void) { return 1; }
#endif
