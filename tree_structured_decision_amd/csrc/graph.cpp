// Graph buckets: one recorded hipGraph per metadata capacity (bucket) runs the
// attention layer and the forked Gated DeltaNet layer for whatever tree was
// last built into the bucket's blob (Flide, kongchang.com page, section
// "pre-recorded execution graphs": a compact set of recorded graphs serves
// varied request mixes). Every kernel is persistent and reads its work counts
// from the blob, so a replay needs no host-side shape information.
#include <new>

#include "common.h"

struct fork_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

using namespace fork;

extern "C" {

fork_status fork_graph_create(const fork_meta* m, const fork_graph_args* a, void* stream, fork_graph** out_h) {
  fork_status st = check_meta(m);
  if (st) return st;
  if (!a || !out_h) return fail(FORK_E_ARG, "args and out must be non-null");
  // validate both layers before recording anything (each forward re-checks)
  size_t need = 0;
  st = gdn_fork_workspace(m, a->gH, a->dk, a->dv, a->dt, &need);
  if (st) return st;
  if (!a->gdn_ws || a->gdn_ws_bytes < need) return fail(FORK_E_WORKSPACE, "GDN workspace too small");
  if (!a->q || !a->k || !a->v || !a->o || !a->gq || !a->gk || !a->gv || !a->a || !a->b || !a->go ||
      !a->seg_start_state)
    return fail(FORK_E_ARG, "a required tensor pointer is null");
  if (a->H < 1 || a->Hkv < 1 || a->H % a->Hkv || a->H / a->Hkv != m->caps.gqa_group)
    return fail(FORK_E_ARG, "attention heads do not match the metadata's gqa_group");
  if (a->D != 64 && a->D != 128) return fail(FORK_E_UNSUPPORTED, "head_dim %d unsupported", a->D);
  if (m->caps.kv_heads != 0 && a->Hkv != m->caps.kv_heads)
    return fail(FORK_E_ARG, "attention kv heads do not match the metadata's kv_heads");
  const size_t aneed = attn_workspace_bytes(m->caps, a->D, a->dt);
  if (aneed && (!a->attn_ws || a->attn_ws_bytes < aneed))
    return fail(FORK_E_WORKSPACE, "attention workspace too small");
  if (a->dk != a->dv || (a->dk != 32 && a->dk != 64 && a->dk != 128))
    return fail(FORK_E_UNSUPPORTED, "dk=%d dv=%d unsupported", a->dk, a->dv);
  if (m->caps.ctx_cap > 0 && (!a->kc || !a->vc))
    return fail(FORK_E_ARG, "the bucket allows cached contexts (ctx_cap %d): kc and vc are required",
                m->caps.ctx_cap);
  if (m->caps.ctx_cap == 0 && (a->kc || a->vc))
    return fail(FORK_E_ARG, "kc / vc given but the bucket has no context capacity (ctx_cap 0)");

  hipStream_t s = (hipStream_t)stream;
  hipStream_t own = nullptr;
  if (!s) {  // the legacy null stream cannot be captured
    FORK_HIP_CHECK(hipStreamCreateWithFlags(&own, hipStreamNonBlocking));
    s = own;
  }
  fork_graph* g = new (std::nothrow) fork_graph;
  if (!g) return fail(FORK_E_ARG, "out of host memory");
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    delete g;
    if (own) (void)hipStreamDestroy(own);
    return fail(FORK_E_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  st = launch_attention(m, a->q, a->k, a->v, a->kc, a->vc, a->o, a->lse, a->H, a->Hkv, a->D, a->scale, a->dt,
                        a->attn_ws, s);
  if (st == FORK_OK)
    st = launch_gdn(m, a->gq, a->gk, a->gv, a->a, a->b, a->root_state, a->go, a->seg_start_state,
                    a->seg_final_state, a->gH, a->dk, a->dv, a->gscale, a->dt, a->gdn_ws, a->gdn_ws_bytes, s);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(s, &graph);
  if (own) (void)hipStreamDestroy(own);
  if (st != FORK_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    delete g;
    if (st != FORK_OK) return st;
    return fail(FORK_E_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  }
  e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    delete g;
    return fail(FORK_E_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  g->graph = graph;
  *out_h = g;
  return FORK_OK;
}

fork_status fork_graph_launch(fork_graph* g, void* stream) {
  if (!g || !g->exec) return fail(FORK_E_ARG, "graph is null");
  FORK_HIP_CHECK(hipGraphLaunch(g->exec, (hipStream_t)stream));
  return FORK_OK;
}

fork_status fork_graph_destroy(fork_graph* g) {
  if (!g) return FORK_OK;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
  return FORK_OK;
}

}  // extern "C"
