// Device half of the segment metadata: expansion of the per-segment arrays
// into per-token arrays, and a dense visibility mask for tests.
//
// Per token t of segment s: tok_seg = s, tok_pos = t - seg_start[s],
// tok_iso_pos = ctx_len[root] + anc_len[s] + tok_pos, the token's position in
// the isolated root-to-segment sequence, after its root's resumed context
// (where a positional encoding would place it).
#include "common.h"

namespace fork {

// One workgroup per segment (grid-stride); threads stride over its tokens.
__global__ void __launch_bounds__(256) meta_expand_kernel(int32_t* __restrict__ blob, BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const int32_t* hdr = blob;
  const int S = hdr[MH_S];
  const int32_t* seg_len = blob + hdr[MH_OFF_SEGLEN];
  const int32_t* seg_start = blob + hdr[MH_OFF_SEGSTART];
  const int32_t* anc_len = blob + hdr[MH_OFF_ANCLEN];
  const int32_t* root = blob + hdr[MH_OFF_ROOT];
  const int32_t* ctx_len = blob + hdr[MH_OFF_CTXLEN];
  int32_t* tok_seg = blob + hdr[MH_OFF_TOKSEG];
  int32_t* tok_pos = blob + hdr[MH_OFF_TOKPOS];
  int32_t* tok_iso = blob + hdr[MH_OFF_TOKISO];
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const int st = seg_start[s], L = seg_len[s], al = ctx_len[root[s]] + anc_len[s];
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      tok_seg[st + i] = s;
      tok_pos[st + i] = i;
      tok_iso[st + i] = al + i;
    }
  }
}

// Token t sees token j iff j is in t's segment at or before t, or j's segment
// is an ancestor of t's segment.
__device__ inline bool visible(const int32_t* blob, int t, int j) {
  const int32_t* hdr = blob;
  const int32_t* tok_seg = blob + hdr[MH_OFF_TOKSEG];
  const int32_t* parent = blob + hdr[MH_OFF_PARENT];
  const int st = tok_seg[t], sj = tok_seg[j];
  if (st == sj) return j <= t;
  for (int p = parent[st]; p >= 0; p = parent[p])
    if (p == sj) return true;
  return false;
}

__global__ void __launch_bounds__(256) dense_mask_kernel(const int32_t* __restrict__ blob,
                                                         uint8_t* __restrict__ mask, BlobGuard guard) {
  if (!blob_ok(blob, guard)) return;
  const int T = blob[MH_T];
  const int64_t n = (int64_t)T * T;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / T), j = (int)(i % T);
    mask[i] = visible(blob, t, j) ? 1 : 0;
  }
}

fork_status launch_meta_expand(const fork_meta* m, hipStream_t stream) {
  // Under graph capture the tree may change between replays: size the grid for
  // the capacity.
  const int S = stream_capturing(stream) ? m->caps.s_cap : m->num_segments;
  const int grid = S < 4096 ? S : 4096;
  hipLaunchKernelGGL(meta_expand_kernel, dim3(grid), dim3(256), 0, stream, (int32_t*)m->dev, blob_guard(m->caps));
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

fork_status launch_dense_mask(const fork_meta* m, uint8_t* mask, hipStream_t stream) {
  const int64_t n = (int64_t)m->num_tokens * m->num_tokens;
  int64_t grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  // the mask holds the descriptor's T x T entries: the blob's tree must not be larger
  BlobGuard g = blob_guard(m->caps);
  g.t_cap = m->num_tokens;
  hipLaunchKernelGGL(dense_mask_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const int32_t*)m->dev, mask, g);
  FORK_HIP_CHECK(hipGetLastError());
  return FORK_OK;
}

}  // namespace fork
