// Host half of the ForkAttention library: tree validation, the metadata plan
// (segment arrays and work lists laid out for one upload), argument checks and
// the public C ABI entry points declared in include/fork.h.
//
// The tree is held as GPU-resident indices over one flattened token stream,
// not as duplicated graphs or re-batched requests (Flide, kongchang.com page,
// section "ForkAttention: exact forking in GPU indices").
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace fork {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

fork_status fail(fork_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
  return st == hipStreamCaptureStatusActive;
}

static fork_status check_caps(const fork_caps* c) {
  if (!c) return fail(FORK_E_ARG, "caps is null");
  if (c->t_cap < 1 || c->t_cap > (1 << 29)) return fail(FORK_E_ARG, "t_cap %d out of range [1, 2^29]", c->t_cap);
  if (c->s_cap < 1 || c->s_cap > (1 << 24)) return fail(FORK_E_ARG, "s_cap %d out of range [1, 2^24]", c->s_cap);
  if (c->depth_cap < 0 || c->depth_cap > kMaxDepthCap)
    return fail(FORK_E_ARG, "depth_cap %d out of range [0, %d]", c->depth_cap, kMaxDepthCap);
  if (c->gqa_group < 1 || c->gqa_group > kAttnRows)
    return fail(FORK_E_UNSUPPORTED, "gqa_group %d out of range [1, %d]", c->gqa_group, kAttnRows);
  if (c->kv_heads < 0 || c->kv_heads > kMaxPartSlots)
    return fail(FORK_E_ARG, "kv_heads %d out of range [0, %d]", c->kv_heads, kMaxPartSlots);
  if (c->ctx_cap < 0 || c->ctx_cap > (1 << 29))
    return fail(FORK_E_ARG, "ctx_cap %d out of range [0, 2^29]", c->ctx_cap);
  // the header stores the arrays' word offsets (and the kernels index the
  // blob) in int32: the whole blob must stay below 2^31 words
  const BlobLayout L = blob_layout(*c);
  if (L.total_words >= ((int64_t)1 << 31))
    return fail(FORK_E_CAPACITY, "capacities t_cap %d, s_cap %d, gqa_group %d need a blob of %lld words (limit 2^31)",
                c->t_cap, c->s_cap, c->gqa_group, (long long)L.total_words);
  return FORK_OK;
}

fork_status check_meta(const fork_meta* m) {
  if (!m) return fail(FORK_E_ARG, "meta is null");
  fork_status st = check_caps(&m->caps);
  if (st) return st;
  if (!m->dev) return fail(FORK_E_ARG, "meta has no device blob (built with fork_meta_plan?)");
  BlobLayout L = blob_layout(m->caps);
  if (m->dev_bytes < (size_t)L.total_words * 4) return fail(FORK_E_WORKSPACE, "device blob too small");
  if (m->num_tokens < 1 || m->num_tokens > m->caps.t_cap || m->num_segments < 1 ||
      m->num_segments > m->caps.s_cap || m->max_depth > m->caps.depth_cap)
    return fail(FORK_E_ARG, "meta descriptor counts are inconsistent with its capacities");
  return FORK_OK;
}

// ---------------------------------------------------------------------------
// The plan: everything the kernels need that depends on the tree only.
static fork_status plan_impl(const int32_t* parent, const int32_t* seg_len, const int32_t* ctx_start_in,
                             const int32_t* ctx_len_in, int32_t S, const fork_caps* caps, void* staging,
                             size_t staging_bytes, size_t* upload_bytes, fork_meta* out) {
  fork_status st = check_caps(caps);
  if (st) return st;
  if (!parent || !seg_len || !staging || !out) return fail(FORK_E_ARG, "null pointer argument");
  if (S < 1) return fail(FORK_E_TREE, "a tree needs at least one segment (got %d)", S);
  if (S > caps->s_cap) return fail(FORK_E_CAPACITY, "%d segments exceed s_cap %d", S, caps->s_cap);
  const BlobLayout L = blob_layout(*caps);
  if (staging_bytes < (size_t)L.upload_cap_words * 4)
    return fail(FORK_E_WORKSPACE, "staging buffer holds %zu bytes, needs %lld", staging_bytes,
                (long long)L.upload_cap_words * 4);

  // validate: parent before child, positive lengths, depth and token capacity
  std::vector<int32_t> depth(S), start(S), root(S), anc(S), root_ord(S, -1), first_child(S, -1);
  int64_t T = 0;
  int32_t max_depth = 0, R = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t p = parent[s];
    if (seg_len[s] < 1) return fail(FORK_E_TREE, "segment %d has length %d (must be >= 1)", s, seg_len[s]);
    if (p < -1 || p >= s)
      return fail(FORK_E_TREE, "segment %d has parent %d (must be -1 or in [0, %d))", s, p, s);
    start[s] = (int32_t)T;
    T += seg_len[s];
    if (T > caps->t_cap) return fail(FORK_E_CAPACITY, "stream exceeds t_cap %d tokens", caps->t_cap);
    if (p < 0) {
      depth[s] = 0;
      root[s] = s;
      anc[s] = 0;
      root_ord[s] = R++;
    } else {
      depth[s] = depth[p] + 1;
      root[s] = root[p];
      anc[s] = anc[p] + seg_len[p];
      if (first_child[p] < 0) first_child[p] = s;
    }
    if (depth[s] > caps->depth_cap)
      return fail(FORK_E_CAPACITY, "segment %d has depth %d > depth_cap %d", s, depth[s], caps->depth_cap);
    max_depth = std::max(max_depth, depth[s]);
  }

  // resumed contexts: cache rows [ctx_start, ctx_start + ctx_len) of a root
  if ((ctx_start_in == nullptr) != (ctx_len_in == nullptr))
    return fail(FORK_E_ARG, "ctx_start and ctx_len must both be given or both be null");
  std::vector<int32_t> ctx_start(S, 0), ctx_len(S, 0);
  int32_t nctx = 0;
  if (ctx_len_in) {
    for (int32_t s = 0; s < S; ++s) {
      const int32_t c0 = ctx_start_in[s], n = ctx_len_in[s];
      if (n < 0) return fail(FORK_E_ARG, "segment %d has context length %d", s, n);
      if (n == 0) continue;
      if (parent[s] >= 0) return fail(FORK_E_TREE, "segment %d has a context but is not a root", s);
      if (c0 < 0 || (int64_t)c0 + n > caps->ctx_cap)
        return fail(FORK_E_CAPACITY, "context rows [%d, %lld) of root %d exceed ctx_cap %d", c0,
                    (long long)c0 + n, s, caps->ctx_cap);
      ctx_start[s] = c0;
      ctx_len[s] = n;
      ++nctx;
    }
  }

  // GDN chunks: never cross a segment boundary; the last one may be partial
  std::vector<int32_t> chunk_base(S);
  int64_t nchunks = 0;
  for (int32_t s = 0; s < S; ++s) {
    chunk_base[s] = (int32_t)nchunks;
    nchunks += (seg_len[s] + kChunk - 1) / kChunk;
  }

  // GDN levels: segments by depth, longest first within a depth (stable)
  std::vector<int32_t> level_off(max_depth + 2, 0), level_seg(S);
  for (int32_t s = 0; s < S; ++s) level_off[depth[s] + 1]++;
  for (int32_t d = 0; d <= max_depth; ++d) level_off[d + 1] += level_off[d];
  {
    std::vector<int32_t> fill(level_off.begin(), level_off.end() - 1);
    for (int32_t s = 0; s < S; ++s) level_seg[fill[depth[s]]++] = s;
    for (int32_t d = 0; d <= max_depth; ++d)
      std::stable_sort(level_seg.begin() + level_off[d], level_seg.begin() + level_off[d + 1],
                       [&](int32_t x, int32_t y) { return seg_len[x] > seg_len[y]; });
  }
  std::vector<int32_t> level_long(max_depth + 1, 0);
  for (int32_t s = 0; s < S; ++s)
    if (seg_len[s] > kChunk) level_long[depth[s]]++;

  // Attention query tiles. Short non-root siblings that follow each other in
  // the stream share their ancestor keys, so they are packed into common
  // tiles: every staged ancestor key/value tile then serves all their rows.
  // A tile's work is measured in 64-key tiles: its ancestors' and its root's
  // context's (anc_kt) plus its own range's.
  const int32_t TT = L.tile_tokens;
  std::vector<int64_t> anc_kt(S);
  for (int32_t s = 0; s < S; ++s)
    anc_kt[s] = parent[s] < 0 ? (ctx_len[s] + kAttnKeys - 1) / kAttnKeys
                              : anc_kt[parent[s]] + (seg_len[parent[s]] + kAttnKeys - 1) / kAttnKeys;
  std::vector<AttnTile> tiles;
  std::vector<int64_t> ktiles;
  tiles.reserve((size_t)(T / TT + S));
  ktiles.reserve(tiles.capacity());
  auto packable = [&](int32_t s) { return parent[s] >= 0 && seg_len[s] < TT; };
  for (int32_t s = 0; s < S;) {
    int32_t e = s + 1;
    if (packable(s))
      while (e < S && packable(e) && parent[e] == parent[s]) ++e;
    const int32_t lo = start[s], hi = start[e - 1] + seg_len[e - 1];
    int32_t seg_of_t0 = s;
    for (int32_t t0 = lo; t0 < hi; t0 += TT) {
      const int32_t t1 = std::min(hi, t0 + TT);
      while (start[seg_of_t0] + seg_len[seg_of_t0] <= t0) ++seg_of_t0;
      int32_t seg_last = seg_of_t0;
      while (start[seg_last] + seg_len[seg_last] < t1) ++seg_last;
      AttnTile tl;
      tl.t0 = t0;
      tl.t1 = t1;
      tl.own_lo = start[seg_of_t0];
      tl.info = (parent[s] + 1) | (seg_last != seg_of_t0 ? kTileMulti : 0);
      tl.kt0 = 0;
      tl.kt1 = (int32_t)(anc_kt[s] + (t1 - tl.own_lo + kAttnKeys - 1) / kAttnKeys);
      tl.slot = -1;
      tl.root = root[s];
      tiles.push_back(tl);
      ktiles.push_back(tl.kt1);
    }
    s = e;
  }

  // Split plan: when the tiles are too few to keep every resident workgroup
  // busy, a tile whose key-tile count exceeds the share P = total /
  // kAttnSlots is cut into parts of about P key tiles; each part writes a partial
  // result (normalised output and log-sum-exp per row) that a merge pass
  // combines. P doubles until the partial slots fit the workspace.
  const int64_t Hkv = caps->kv_heads;
  int64_t P = INT64_MAX;
  auto nparts_of = [&](int64_t kt) -> int64_t {
    return kt > P ? std::min<int64_t>(kMaxSplit, (kt + P - 1) / P) : 1;
  };
  if (Hkv > 0) {
    int64_t W = 0;
    for (int64_t kt : ktiles) W += kt * Hkv;
    P = std::max<int64_t>(kMinPartTiles, (W + kAttnSlots - 1) / kAttnSlots);
    for (;;) {
      int64_t slots = 0, groups = 0;
      for (int64_t kt : ktiles)
        if (nparts_of(kt) > 1) {
          slots += nparts_of(kt);
          ++groups;
        }
      if (slots * Hkv <= kMaxPartSlots && groups <= L.merge_cap) break;
      P *= 2;
    }
  }
  std::vector<AttnTile> entries;
  std::vector<int64_t> cost;
  std::vector<AttnMerge> merges;
  int32_t nslots = 0;
  for (size_t i = 0; i < tiles.size(); ++i) {
    const int64_t kt = ktiles[i], n = nparts_of(kt);
    if (n == 1) {
      entries.push_back(tiles[i]);
      cost.push_back(kt);
      continue;
    }
    AttnMerge mg;
    mg.t0 = tiles[i].t0;
    mg.t1 = tiles[i].t1;
    mg.nparts = (int32_t)n;
    mg.slot0 = nslots;
    merges.push_back(mg);
    for (int64_t p = 0; p < n; ++p) {
      AttnTile e = tiles[i];
      e.kt0 = (int32_t)(kt * p / n);
      e.kt1 = (int32_t)(kt * (p + 1) / n);
      e.slot = nslots + (int32_t)p;
      entries.push_back(e);
      cost.push_back(e.kt1 - e.kt0);
    }
    nslots += (int32_t)n;
  }
  if ((int64_t)entries.size() > L.tile_cap) return fail(FORK_E_CAPACITY, "tile list overflow");
  // most expensive first (counting sort on key tiles, stable)
  std::vector<AttnTile> sorted(entries.size());
  {
    int64_t maxc = 0;
    for (int64_t c : cost) maxc = std::max(maxc, c);
    const int64_t nb = maxc + 1;
    std::vector<int64_t> cnt(nb + 1, 0);
    for (int64_t c : cost) cnt[maxc - c]++;
    int64_t acc = 0;
    for (int64_t i = 0; i <= nb; ++i) {
      int64_t x = cnt[i];
      cnt[i] = acc;
      acc += x;
    }
    for (size_t i = 0; i < entries.size(); ++i) sorted[cnt[maxc - cost[i]]++] = entries[i];
  }

  // lay out the upload region
  int32_t* w = (int32_t*)staging;
  memset(w, 0, MH_WORDS * 4);
  int64_t off = MH_WORDS;
  auto put = [&](int hdr_slot, const int32_t* src, int64_t n) {
    off = (off + 3) & ~int64_t(3);
    w[hdr_slot] = (int32_t)off;
    if (n) memcpy(w + off, src, (size_t)n * 4);
    off += n;
  };
  put(MH_OFF_PARENT, parent, S);
  put(MH_OFF_SEGLEN, seg_len, S);
  put(MH_OFF_SEGSTART, start.data(), S);
  put(MH_OFF_DEPTH, depth.data(), S);
  put(MH_OFF_ROOT, root.data(), S);
  put(MH_OFF_ROOTORD, root_ord.data(), S);
  put(MH_OFF_ANCLEN, anc.data(), S);
  put(MH_OFF_FIRSTCHILD, first_child.data(), S);
  put(MH_OFF_CHUNKBASE, chunk_base.data(), S);
  put(MH_OFF_LEVELOFF, level_off.data(), max_depth + 2);
  put(MH_OFF_LEVELSEG, level_seg.data(), S);
  put(MH_OFF_LEVELLONG, level_long.data(), max_depth + 1);
  put(MH_OFF_CTXSTART, ctx_start.data(), S);
  put(MH_OFF_CTXLEN, ctx_len.data(), S);
  {
    off = (off + 3) & ~int64_t(3);
    w[MH_OFF_CHUNKS] = (int32_t)off;
    for (int32_t s = 0; s < S; ++s)
      for (int32_t c0 = 0; c0 < seg_len[s]; c0 += kChunk) {
        w[off++] = start[s] + c0;
        w[off++] = std::min(kChunk, seg_len[s] - c0);
      }
  }
  {
    // the scan items' records (GdnRec): one per segment in level order, and
    // the packed list (runs of consecutive leaf siblings of at most a chunk
    // in total share a record), longest first within each depth
    auto src_of = [&](int32_t s) { return parent[s] < 0 ? -1 - root_ord[s] : first_child[parent[s]]; };
    std::vector<GdnRec> rec(S);
    for (int32_t i = 0; i < S; ++i) {
      const int32_t s = level_seg[i];
      rec[i] = GdnRec{s, start[s], seg_len[s], src_of(s), first_child[s], 1, 0, 0};
    }
    put(MH_OFF_GDNREC, (const int32_t*)rec.data(), (int64_t)S * kGdnRecWords);
    auto leaf = [&](int32_t s) { return parent[s] >= 0 && first_child[s] < 0 && seg_len[s] <= kChunk; };
    std::vector<GdnRec> packs;
    std::vector<int32_t> pack_depth;
    for (int32_t s = 0; s < S; ++s) {
      if (leaf(s) && !packs.empty() && packs.back().seg + packs.back().nsib == s && packs.back().nsib > 0 &&
          parent[packs.back().seg] == parent[s] && leaf(packs.back().seg) &&
          packs.back().len + seg_len[s] <= kChunk) {
        packs.back().len += seg_len[s];
        packs.back().nsib += 1;
        continue;
      }
      packs.push_back(GdnRec{s, start[s], seg_len[s], src_of(s), first_child[s], 1, 0, 0});
      pack_depth.push_back(depth[s]);
    }
    std::vector<int32_t> pack_off(max_depth + 2, 0), order(packs.size());
    for (int32_t d : pack_depth) pack_off[d + 1]++;
    for (int32_t d = 0; d <= max_depth; ++d) pack_off[d + 1] += pack_off[d];
    {
      std::vector<int32_t> fill(pack_off.begin(), pack_off.end() - 1);
      for (size_t i = 0; i < packs.size(); ++i) order[fill[pack_depth[i]]++] = (int32_t)i;
      for (int32_t d = 0; d <= max_depth; ++d)
        std::stable_sort(order.begin() + pack_off[d], order.begin() + pack_off[d + 1],
                         [&](int32_t x, int32_t y) { return packs[x].len > packs[y].len; });
    }
    std::vector<GdnRec> sorted_packs(packs.size());
    for (size_t i = 0; i < packs.size(); ++i) sorted_packs[i] = packs[order[i]];
    put(MH_OFF_GDNPACK, (const int32_t*)sorted_packs.data(), (int64_t)sorted_packs.size() * kGdnRecWords);
    put(MH_OFF_PACKOFF, pack_off.data(), max_depth + 2);
  }
  put(MH_OFF_TILES, (const int32_t*)sorted.data(), (int64_t)sorted.size() * 8);
  put(MH_OFF_MERGE, (const int32_t*)merges.data(), (int64_t)merges.size() * 4);
  if (off > L.upload_cap_words) return fail(FORK_E_CAPACITY, "metadata upload region overflow");
  const int64_t tstride = ((int64_t)caps->t_cap + 63) / 64 * 64;
  w[MH_MAGIC] = kMetaMagic;
  w[MH_T] = (int32_t)T;
  w[MH_S] = S;
  w[MH_R] = R;
  w[MH_MAXDEPTH] = max_depth;
  w[MH_NTILES] = (int32_t)sorted.size();
  w[MH_NCHUNKS] = (int32_t)nchunks;
  w[MH_TILE_TOKENS] = TT;
  w[MH_GQA] = caps->gqa_group;
  w[MH_OFF_TOKSEG] = (int32_t)L.tok_off_words;
  w[MH_OFF_TOKPOS] = (int32_t)(L.tok_off_words + tstride);
  w[MH_OFF_TOKISO] = (int32_t)(L.tok_off_words + 2 * tstride);
  w[MH_UPLOAD_WORDS] = (int32_t)off;
  w[MH_NMERGE] = (int32_t)merges.size();
  w[MH_NPARTS] = nslots;
  w[MH_KV_HEADS] = (int32_t)Hkv;
  w[MH_NCTX] = nctx;

  memset(out, 0, sizeof(*out));
  out->num_tokens = (int32_t)T;
  out->num_segments = S;
  out->num_roots = R;
  out->max_depth = max_depth;
  out->num_attn_tiles = (int32_t)sorted.size();
  out->num_chunks = (int32_t)nchunks;
  out->tile_tokens = TT;
  out->num_attn_merges = (int32_t)merges.size();
  out->num_attn_parts = nslots;
  out->caps = *caps;
  for (int32_t d = 0; d <= max_depth && d < FORK_PLAN_DEPTHS; ++d) {
    out->level_segs[d] = level_off[d + 1] - level_off[d];
    out->level_long[d] = level_long[d];
  }
  if (upload_bytes) *upload_bytes = (size_t)off * 4;
  return FORK_OK;
}

}  // namespace fork

using namespace fork;

extern "C" {

const char* fork_last_error(void) { return g_err; }

const char* fork_version(void) { return "forkattn-gfx950 0.1"; }

fork_status fork_meta_size(const fork_caps* caps_h, size_t* dev_bytes_h, size_t* staging_bytes_h) {
  g_err[0] = 0;
  fork_status st = check_caps(caps_h);
  if (st) return st;
  BlobLayout L = blob_layout(*caps_h);
  if (dev_bytes_h) *dev_bytes_h = (size_t)L.total_words * 4;
  if (staging_bytes_h) *staging_bytes_h = (size_t)L.upload_cap_words * 4;
  return FORK_OK;
}

fork_status fork_meta_plan_ctx(const int32_t* parent_h, const int32_t* seg_len_h, const int32_t* ctx_start_h,
                               const int32_t* ctx_len_h, int32_t num_segments, const fork_caps* caps_h,
                               void* staging_h, size_t staging_bytes, size_t* upload_bytes_h,
                               fork_meta* out_h) {
  g_err[0] = 0;
  return plan_impl(parent_h, seg_len_h, ctx_start_h, ctx_len_h, num_segments, caps_h, staging_h,
                   staging_bytes, upload_bytes_h, out_h);
}

fork_status fork_meta_plan(const int32_t* parent_h, const int32_t* seg_len_h, int32_t num_segments,
                           const fork_caps* caps_h, void* staging_h, size_t staging_bytes,
                           size_t* upload_bytes_h, fork_meta* out_h) {
  return fork_meta_plan_ctx(parent_h, seg_len_h, nullptr, nullptr, num_segments, caps_h, staging_h,
                            staging_bytes, upload_bytes_h, out_h);
}

fork_status fork_meta_build(const int32_t* parent_h, const int32_t* seg_len_h, int32_t num_segments,
                            const fork_caps* caps_h, void* dev, size_t dev_bytes, void* staging_h,
                            size_t staging_bytes, fork_meta* out_h, void* stream) {
  return fork_meta_build_ctx(parent_h, seg_len_h, nullptr, nullptr, num_segments, caps_h, dev, dev_bytes,
                             staging_h, staging_bytes, out_h, stream);
}

fork_status fork_meta_build_ctx(const int32_t* parent_h, const int32_t* seg_len_h, const int32_t* ctx_start_h,
                                const int32_t* ctx_len_h, int32_t num_segments, const fork_caps* caps_h,
                                void* dev, size_t dev_bytes, void* staging_h, size_t staging_bytes,
                                fork_meta* out_h, void* stream) {
  g_err[0] = 0;
  if (!dev) return fail(FORK_E_ARG, "dev is null");
  fork_status st = check_caps(caps_h);
  if (st) return st;
  BlobLayout L = blob_layout(*caps_h);
  if (dev_bytes < (size_t)L.total_words * 4)
    return fail(FORK_E_WORKSPACE, "device blob holds %zu bytes, needs %lld", dev_bytes,
                (long long)L.total_words * 4);
  fork_meta m;
  size_t up = 0;
  st = plan_impl(parent_h, seg_len_h, ctx_start_h, ctx_len_h, num_segments, caps_h, staging_h, staging_bytes,
                 &up, &m);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  FORK_HIP_CHECK(hipMemcpyAsync(dev, staging_h, up, hipMemcpyHostToDevice, s));
  m.dev = dev;
  m.dev_bytes = dev_bytes;
  st = launch_meta_expand(&m, s);
  if (st) return st;
  *out_h = m;
  return FORK_OK;
}

fork_status fork_meta_export(const fork_meta* m, int32_t array_id, int32_t* dst_h, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!dst_h) return fail(FORK_E_ARG, "dst is null");
  hipStream_t s = (hipStream_t)stream;
  int32_t hdr[MH_WORDS];
  FORK_HIP_CHECK(hipMemcpyAsync(hdr, m->dev, sizeof(hdr), hipMemcpyDeviceToHost, s));
  FORK_HIP_CHECK(hipStreamSynchronize(s));
  int slot;
  int64_t n;
  switch (array_id) {
    case FORK_ARR_TOK_SEG: slot = MH_OFF_TOKSEG; n = hdr[MH_T]; break;
    case FORK_ARR_TOK_POS: slot = MH_OFF_TOKPOS; n = hdr[MH_T]; break;
    case FORK_ARR_TOK_ISO_POS: slot = MH_OFF_TOKISO; n = hdr[MH_T]; break;
    case FORK_ARR_SEG_START: slot = MH_OFF_SEGSTART; n = hdr[MH_S]; break;
    case FORK_ARR_DEPTH: slot = MH_OFF_DEPTH; n = hdr[MH_S]; break;
    case FORK_ARR_ANC_LEN: slot = MH_OFF_ANCLEN; n = hdr[MH_S]; break;
    case FORK_ARR_ROOT: slot = MH_OFF_ROOT; n = hdr[MH_S]; break;
    case FORK_ARR_CTX_START: slot = MH_OFF_CTXSTART; n = hdr[MH_S]; break;
    case FORK_ARR_CTX_LEN: slot = MH_OFF_CTXLEN; n = hdr[MH_S]; break;
    default: return fail(FORK_E_ARG, "unknown array id %d", array_id);
  }
  FORK_HIP_CHECK(hipMemcpyAsync(dst_h, (const int32_t*)m->dev + hdr[slot], (size_t)n * 4,
                                hipMemcpyDeviceToHost, s));
  FORK_HIP_CHECK(hipStreamSynchronize(s));
  return FORK_OK;
}

fork_status fork_meta_check(const fork_meta* m, int32_t* device_error_h, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  int32_t word = 0;
  FORK_HIP_CHECK(hipMemcpyAsync(&word, (const int32_t*)m->dev + kErrWord, sizeof(word), hipMemcpyDeviceToHost, s));
  FORK_HIP_CHECK(hipStreamSynchronize(s));
  if (device_error_h) *device_error_h = word;
  if (word == 0) return FORK_OK;
  return fail(FORK_E_DEVICE, "a kernel stopped on this blob: %s%s(device error word 0x%x)",
              (word & FORK_DEVERR_MAGIC) ? "it holds no built metadata; " : "",
              (word & FORK_DEVERR_CAPACITY) ? "its tree exceeds the capacities the launch was made for; " : "",
              (unsigned)word);
}

fork_status fork_meta_dense_mask(const fork_meta* m, uint8_t* mask, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!mask) return fail(FORK_E_ARG, "mask is null");
  if (m->num_tokens > 8192) return fail(FORK_E_ARG, "dense mask limited to T <= 8192");
  return launch_dense_mask(m, mask, (hipStream_t)stream);
}

fork_status fork_attn_workspace(const fork_meta* m, int32_t H, int32_t Hkv, int32_t D, fork_dtype dt,
                                size_t* bytes_h) {
  g_err[0] = 0;
  fork_status st = check_caps(m ? &m->caps : nullptr);
  if (st) return st;
  if (!bytes_h) return fail(FORK_E_ARG, "bytes_h is null");
  (void)H; (void)Hkv; (void)dt;
  if (D != 64 && D != 128) return fail(FORK_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", D);
  *bytes_h = attn_workspace_bytes(m->caps, D, dt);
  return FORK_OK;
}

fork_status fork_attn_forward(const fork_meta* m, const void* q, const void* k, const void* v, void* o,
                              float* lse, int32_t H, int32_t Hkv, int32_t D, float scale,
                              fork_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  return fork_attn_forward_ctx(m, q, k, v, nullptr, nullptr, o, lse, H, Hkv, D, scale, dt, ws, ws_bytes,
                               stream);
}

}  // extern "C"

// Argument checks shared by the attention entry points (everything but the workspace).
static fork_status check_attn_args(const fork_meta* m, const void* q, const void* k, const void* v,
                                   const void* kc, const void* vc, const void* o, int32_t H, int32_t Hkv,
                                   int32_t D, fork_dtype dt) {
  fork_status st = check_meta(m);
  if (st) return st;
  if (!q || !k || !v || !o) return fail(FORK_E_ARG, "q, k, v and o must be non-null");
  if (m->caps.ctx_cap > 0 && (!kc || !vc))
    return fail(FORK_E_ARG, "the metadata was built for cached contexts (ctx_cap %d): kc and vc are required",
                m->caps.ctx_cap);
  if (m->caps.ctx_cap == 0 && (kc || vc))
    return fail(FORK_E_ARG, "kc / vc given but the metadata has no context capacity (ctx_cap 0)");
  if (H < 1 || Hkv < 1 || H % Hkv) return fail(FORK_E_ARG, "H=%d must be a positive multiple of Hkv=%d", H, Hkv);
  if (H / Hkv != m->caps.gqa_group)
    return fail(FORK_E_ARG, "H/Hkv=%d differs from the gqa_group %d the metadata was built for", H / Hkv,
                m->caps.gqa_group);
  if (D != 64 && D != 128) return fail(FORK_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", D);
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (m->caps.kv_heads != 0 && Hkv != m->caps.kv_heads)
    return fail(FORK_E_ARG, "Hkv=%d differs from the kv_heads %d the metadata was built for", Hkv,
                m->caps.kv_heads);
  return FORK_OK;
}

extern "C" {

fork_status fork_attn_forward_ctx(const fork_meta* m, const void* q, const void* k, const void* v,
                                  const void* kc, const void* vc, void* o, float* lse, int32_t H,
                                  int32_t Hkv, int32_t D, float scale, fork_dtype dt, void* ws,
                                  size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  fork_status st = check_attn_args(m, q, k, v, kc, vc, o, H, Hkv, D, dt);
  if (st) return st;
  const size_t need = attn_workspace_bytes(m->caps, D, dt);
  if (need && (!ws || ws_bytes < need))
    return fail(FORK_E_WORKSPACE, "attention workspace holds %zu bytes, needs %zu", ws_bytes, need);
  return launch_attention(m, q, k, v, kc, vc, o, lse, H, Hkv, D, scale, dt, ws, (hipStream_t)stream);
}

fork_status fork_attn_forward_qk8(const fork_meta* m, const void* q8, const float* q_scale, const void* k8,
                                  const float* k_scale, const void* v, void* o, float* lse, int32_t H,
                                  int32_t Hkv, int32_t D, float scale, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  fork_status st = check_attn_args(m, q8, k8, v, nullptr, nullptr, o, H, Hkv, D, FORK_BF16);
  if (st) return st;
  if (!q_scale || !k_scale) return fail(FORK_E_ARG, "q_scale and k_scale must be non-null");
  if (D != 128) return fail(FORK_E_UNSUPPORTED, "FP8 scores need head_dim 128 (got %d)", D);
  if (m->caps.ctx_cap != 0)
    return fail(FORK_E_UNSUPPORTED, "FP8 scores are not supported with cached contexts (ctx_cap %d)", m->caps.ctx_cap);
  if ((uintptr_t)q8 % 16 || (uintptr_t)k8 % 16) return fail(FORK_E_ARG, "q8 and k8 must be 16-byte aligned");
  const size_t need = attn_workspace_bytes(m->caps, D, FORK_BF16);
  if (need && (!ws || ws_bytes < need))
    return fail(FORK_E_WORKSPACE, "attention workspace holds %zu bytes, needs %zu", ws_bytes, need);
  return launch_attention_any(m, q8, q_scale, k8, k_scale, v, nullptr, nullptr, o, lse, H, Hkv, D, scale, FORK_BF16,
                              ws, (hipStream_t)stream);
}

fork_status fork_attn_forward_noalloc(const fork_meta* m, const void* q, const void* k, const void* v,
                                      const void* kc, const void* vc, void* o, float* lse, int32_t H,
                                      int32_t Hkv, int32_t D, float scale, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_attn_args(m, q, k, v, kc, vc, o, H, Hkv, D, dt);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  // the slots this launch may touch: the tree's split plan, or under capture
  // (the tree may change between replays) every slot the blob can plan
  const size_t slot = attn_slot_bytes(D, dt);
  const int64_t parts = m->caps.kv_heads == 0 ? 0 : (stream_capturing(s) ? kMaxPartSlots / Hkv : m->num_attn_parts);
  const size_t need = (size_t)parts * Hkv * slot;
  if (need > FORK_ATTN_SCRATCH_BYTES)
    return fail(FORK_E_CAPACITY, "split query tiles need %zu bytes of partial results; the scratch array holds %zu",
                need, (size_t)FORK_ATTN_SCRATCH_BYTES);
  void* scratch = nullptr;
  st = attn_scratch(&scratch);
  if (st) return st;
  return launch_attention(m, q, k, v, kc, vc, o, lse, H, Hkv, D, scale, dt, scratch, s);
}

fork_status gdn_fork_workspace(const fork_meta* m, int32_t H, int32_t dk, int32_t dv, fork_dtype dt,
                               size_t* bytes_h) {
  g_err[0] = 0;
  fork_status st = check_caps(m ? &m->caps : nullptr);
  if (st) return st;
  if (!bytes_h) return fail(FORK_E_ARG, "bytes_h is null");
  if (H < 1 || dk < 1 || dv < 1) return fail(FORK_E_ARG, "bad head shape");
  (void)dt;
  *bytes_h = gdn_workspace_bytes(m, H, dk, dv);
  return FORK_OK;
}

fork_status gdn_fork_forward(const fork_meta* m, const void* q, const void* k, const void* v,
                             const float* a, const float* b, const float* root_state, void* o,
                             float* seg_start_state, float* seg_final_state, int32_t H, int32_t dk,
                             int32_t dv, float scale, fork_dtype dt, void* ws, size_t ws_bytes,
                             void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!q || !k || !v || !a || !b || !o || !seg_start_state)
    return fail(FORK_E_ARG, "q, k, v, a, b, o and seg_start_state must be non-null");
  if (H < 1) return fail(FORK_E_ARG, "H=%d", H);
  if (dk != dv || (dk != 32 && dk != 64 && dk != 128))
    return fail(FORK_E_UNSUPPORTED, "dk=%d dv=%d unsupported (dk == dv in {32, 64, 128})", dk, dv);
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  const size_t need = gdn_workspace_bytes(m, H, dk, dv);
  if (!ws || ws_bytes < need) return fail(FORK_E_WORKSPACE, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
  return launch_gdn(m, q, k, v, a, b, root_state, o, seg_start_state, seg_final_state, H, dk, dv, scale,
                    dt, ws, ws_bytes, (hipStream_t)stream);
}

fork_status gdn_fork_forward_fp8(const fork_meta* m, const void* q8, const float* q_scale, const void* k8,
                                 const float* k_scale, const void* v8, const float* v_scale, const float* a,
                                 const float* b, const float* root_state, void* o, float* seg_start_state,
                                 float* seg_final_state, int32_t H, int32_t dk, int32_t dv, float scale, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !a || !b || !o || !seg_start_state)
    return fail(FORK_E_ARG, "q8, k8, v8, their scales, a, b, o and seg_start_state must be non-null");
  if (H < 1) return fail(FORK_E_ARG, "H=%d", H);
  if (dk != 128 || dv != 128) return fail(FORK_E_UNSUPPORTED, "FP8 inputs need dk = dv = 128 (got %d, %d)", dk, dv);
  if ((uintptr_t)q8 % 16 || (uintptr_t)k8 % 16 || (uintptr_t)v8 % 16)
    return fail(FORK_E_ARG, "q8, k8 and v8 must be 16-byte aligned");
  return launch_gdn_fp8(m, q8, q_scale, k8, k_scale, v8, v_scale, a, b, root_state, o, seg_start_state,
                        seg_final_state, H, scale, (hipStream_t)stream);
}

fork_status fork_rope_forward(const fork_meta* m, void* x, int32_t nheads, int32_t D, float theta,
                              fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!x) return fail(FORK_E_ARG, "x is null");
  if (nheads < 1) return fail(FORK_E_ARG, "nheads=%d", nheads);
  if (D < 8 || D > 256 || D % 8) return fail(FORK_E_UNSUPPORTED, "rotary dim %d unsupported (multiple of 8, 8..256)", D);
  if (!(theta > 1.f)) return fail(FORK_E_ARG, "theta must be > 1");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_rope(m, x, (long long)nheads * D, x, nheads, D, theta, dt, (hipStream_t)stream);
}

fork_status fork_rope_copy_forward(const fork_meta* m, const void* src, int64_t ld_src, void* dst, int32_t nheads,
                                   int32_t D, float theta, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!src || !dst) return fail(FORK_E_ARG, "src and dst must be non-null");
  if (nheads < 1) return fail(FORK_E_ARG, "nheads=%d", nheads);
  if (D < 8 || D > 256 || D % 8) return fail(FORK_E_UNSUPPORTED, "rotary dim %d unsupported (multiple of 8, 8..256)", D);
  if (ld_src < (int64_t)nheads * D || ld_src % 4) return fail(FORK_E_ARG, "ld_src %lld (>= nheads * D, a multiple of 4)", (long long)ld_src);
  const size_t esz = dt == FORK_BF16 ? 2 : 4;
  if ((uintptr_t)src % (4 * esz) || (uintptr_t)dst % (4 * esz)) return fail(FORK_E_ARG, "src and dst must be aligned to 4 elements");
  if (theta != 0.f && !(theta > 1.f)) return fail(FORK_E_ARG, "theta must be > 1 (or 0: copy)");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  const char* s0 = (const char*)src;
  const char* d0 = (const char*)dst;
  const size_t span = (size_t)m->caps.t_cap * ld_src * esz, dspan = (size_t)m->caps.t_cap * nheads * D * esz;
  if (d0 < s0 + span && s0 < d0 + dspan) return fail(FORK_E_ARG, "src and dst must not overlap");
  return launch_rope(m, src, (long long)ld_src, dst, nheads, D, theta, dt, (hipStream_t)stream);
}

fork_status fork_conv_forward(const fork_meta* m, const void* x, const float* w, const float* bias,
                              const float* conv_state, void* y, int32_t C, int32_t K, int32_t act,
                              fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!x || !w || !y) return fail(FORK_E_ARG, "x, w and y must be non-null");
  if (x == y) return fail(FORK_E_ARG, "x and y must not overlap");
  if ((uintptr_t)w % 16) return fail(FORK_E_ARG, "w must be 16-byte aligned");
  if (C < 8 || C % 8) return fail(FORK_E_UNSUPPORTED, "channels %d unsupported (a positive multiple of 8)", C);
  if (K < 2 || K > 8) return fail(FORK_E_UNSUPPORTED, "kernel width %d unsupported (2..8)", K);
  if (act != 0 && act != 1) return fail(FORK_E_ARG, "act %d (0 identity, 1 SiLU)", act);
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_conv(m, x, w, bias, conv_state, y, C, K, act, dt, (hipStream_t)stream);
}

fork_status fork_gate_forward(const fork_meta* m, const void* x, const void* g, int64_t ld_g, const float* w,
                              void* y, int32_t nheads, int32_t D, int32_t mode, float eps, fork_dtype dt,
                              void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (mode < 0 || mode > 2) return fail(FORK_E_ARG, "mode %d (0 sigmoid gate, 1 gated RMS norm, 2 RMS norm)", mode);
  if (!x || !y) return fail(FORK_E_ARG, "x and y must be non-null");
  if (mode != 2 && !g) return fail(FORK_E_ARG, "mode %d needs the gate g", mode);
  if (mode != 0 && !w) return fail(FORK_E_ARG, "mode %d needs the weight w", mode);
  if (w && (uintptr_t)w % 16) return fail(FORK_E_ARG, "w must be 16-byte aligned");
  if (nheads < 1) return fail(FORK_E_ARG, "nheads=%d", nheads);
  if (D < 8 || D > 65536 || D % 8) return fail(FORK_E_UNSUPPORTED, "row size %d unsupported (multiple of 8, 8..65536)", D);
  if (mode != 0 && !(eps > 0.f)) return fail(FORK_E_ARG, "eps must be > 0");
  if (ld_g == 0) ld_g = (int64_t)nheads * D;
  if (mode != 2 && (ld_g < (int64_t)nheads * D || ld_g % 8))
    return fail(FORK_E_ARG, "ld_g %lld (>= nheads * D, a multiple of 8)", (long long)ld_g);
  if (mode != 2 && (uintptr_t)g % 16) return fail(FORK_E_ARG, "g must be 16-byte aligned");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_gate(m, x, g, (long long)ld_g, w, y, nheads, D, mode, eps, dt, (hipStream_t)stream);
}

fork_status fork_option_readout(const fork_meta* m, const void* x, const float* w, int32_t C, float* score,
                                float* prob, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!x || !w || !score || !prob) return fail(FORK_E_ARG, "x, w, score and prob must be non-null");
  if (C < 8 || C > 65536 || C % 8) return fail(FORK_E_UNSUPPORTED, "row size C=%d unsupported (multiple of 8, 8..65536)", C);
  if ((uintptr_t)x % 16 || (uintptr_t)w % 16) return fail(FORK_E_ARG, "x and w must be 16-byte aligned");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_readout(m, x, w, C, score, prob, dt, (hipStream_t)stream);
}

fork_status gdn_inputs_forward(const fork_meta* m, const void* c, const void* ab, int64_t ld_ab, const float* a_log,
                               const float* dt_bias, void* q, void* k, void* v, float* a, float* b, int32_t H,
                               int32_t dk, int32_t dv, float eps, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!ab || !a_log || !dt_bias || !a || !b) return fail(FORK_E_ARG, "ab, a_log, dt_bias, a and b must be non-null");
  if (c && (!q || !k || !v)) return fail(FORK_E_ARG, "q, k and v must be non-null when c is given");
  if (H < 1) return fail(FORK_E_ARG, "H=%d", H);
  if (dk < 8 || dk > 1024 || dk % 8 || dv < 8 || dv > 1024 || dv % 8)
    return fail(FORK_E_UNSUPPORTED, "head sizes dk=%d dv=%d unsupported (multiples of 8, 8..1024)", dk, dv);
  if (!(eps > 0.f)) return fail(FORK_E_ARG, "eps must be > 0");
  if (ld_ab == 0) ld_ab = 2 * (int64_t)H;
  if (ld_ab < 2 * (int64_t)H) return fail(FORK_E_ARG, "ld_ab %lld < 2 H", (long long)ld_ab);
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_gdn_inputs(m, c, ab, (long long)ld_ab, a_log, dt_bias, q, k, v, a, b, H, dk, dv, eps, dt,
                           (hipStream_t)stream);
}

fork_status gdn_conv_inputs_forward(const fork_meta* m, const void* x, const float* w, const float* bias,
                                    const float* conv_state, void* q, void* k, void* v, int32_t H, int32_t dk,
                                    int32_t dv, int32_t K, float eps, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  fork_status st = check_meta(m);
  if (st) return st;
  if (!x || !w || !q || !k || !v) return fail(FORK_E_ARG, "x, w, q, k and v must be non-null");
  if (H < 1) return fail(FORK_E_ARG, "H=%d", H);
  if (dk != dv || dk < 8 || dk > 512 || (dk & (dk - 1)))
    return fail(FORK_E_UNSUPPORTED, "head sizes dk=%d dv=%d (equal, a power of two in 8..512)", dk, dv);
  if (K < 2 || K > 8) return fail(FORK_E_UNSUPPORTED, "kernel width %d unsupported (2..8)", K);
  if ((uintptr_t)w % 16) return fail(FORK_E_ARG, "w must be 16-byte aligned");
  if (!(eps > 0.f)) return fail(FORK_E_ARG, "eps must be > 0");
  if (x == q || x == k || x == v) return fail(FORK_E_ARG, "x must not overlap the outputs");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_conv_split(m, x, w, bias, conv_state, q, k, v, H, dk, dv, K, eps, dt, (hipStream_t)stream);
}

fork_status fork_linear_forward(const void* x, const void* w, void* y, int32_t M, int32_t N, int32_t K,
                                int32_t accumulate, fork_dtype dt, void* stream) {
  g_err[0] = 0;
  if (!x || !w || !y) return fail(FORK_E_ARG, "x, w and y must be non-null");
  if (M < 1 || N < 1 || K < 1) return fail(FORK_E_ARG, "M=%d N=%d K=%d", M, N, K);
  if (y == x || y == w) return fail(FORK_E_ARG, "y must not overlap x or w");
  if (accumulate != 0 && accumulate != 1) return fail(FORK_E_ARG, "accumulate %d (0 or 1)", accumulate);
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_linear(x, w, y, M, N, K, accumulate, dt, (hipStream_t)stream);
}

fork_status fork_quantize_fp8(const void* x, void* q, float* scales, int64_t rows, int32_t K, fork_dtype dt,
                              void* stream) {
  g_err[0] = 0;
  if (!x || !q || !scales) return fail(FORK_E_ARG, "x, q and scales must be non-null");
  if (rows < 1) return fail(FORK_E_ARG, "rows=%lld", (long long)rows);
  if (K < 8 || K % 8) return fail(FORK_E_UNSUPPORTED, "row length %d (a positive multiple of 8)", K);
  if ((uintptr_t)x % 16 || (uintptr_t)q % 8) return fail(FORK_E_ARG, "x must be 16-byte and q 8-byte aligned");
  if (dt != FORK_F32 && dt != FORK_BF16) return fail(FORK_E_UNSUPPORTED, "unknown dtype %d", (int)dt);
  return launch_quantize_fp8(x, q, scales, (long long)rows, K, dt, (hipStream_t)stream);
}

fork_status fork_linear_fp8_forward(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                                    void* y, int32_t M, int32_t N, int32_t K, int32_t accumulate, void* stream) {
  g_err[0] = 0;
  if (!xq || !x_scale || !wq || !w_scale || !y) return fail(FORK_E_ARG, "every pointer must be non-null");
  if (M < 1 || N < 1 || K < 1) return fail(FORK_E_ARG, "M=%d N=%d K=%d", M, N, K);
  if (K % 16) return fail(FORK_E_UNSUPPORTED, "K=%d (fp8 products need a multiple of 16)", K);
  if (y == xq || y == wq) return fail(FORK_E_ARG, "y must not overlap xq or wq");
  if (accumulate != 0 && accumulate != 1) return fail(FORK_E_ARG, "accumulate %d (0 or 1)", accumulate);
  return launch_linear_fp8(xq, x_scale, wq, w_scale, y, M, N, K, accumulate, (hipStream_t)stream);
}

}  // extern "C"
