// Whole-step decode graph: warm-up, capture and replay of a multi-layer
// decode step as one hipGraph.
//
// Method (AstrAI commit-list pages): [attention_backend.py @47b3ed4], the
// commits adding a graph context with a warm-up -> capture -> replay
// lifecycle, one graph per batch size with every input at a fixed address,
// a live forward run before capture, and a preallocated decode output so the
// captured decode allocates nothing.  Here the captured work is the decode
// calls of all layers of one step (each with the optional fused KV append);
// a replay re-runs them with whatever the fixed buffers hold, including new
// sequence lengths in the device index arrays.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <new>

#include "abi_internal.hpp"
#include "astr_attn.h"

struct astr_decode_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int32_t num_layers = 0;
  int32_t batch = 0;
};

namespace {

using astr::fail;
using astr::ok;

// Enqueues every layer's decode (fused append when new_kv is set) on `stream`.
int enqueue_step(const astr_paged_args* layers, const astr_new_kv* new_kv, int32_t n, void* ws, size_t ws_bytes,
                 void* stream) {
  for (int32_t l = 0; l < n; ++l) {
    const int st = astr::decode_impl(&layers[l], new_kv != nullptr ? &new_kv[l] : nullptr, ws, ws_bytes, stream);
    if (st != ASTR_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "%s", astr::last_error());
      return fail(st, "layer %d: %s", l, msg);
    }
  }
  return ASTR_OK;
}

}  // namespace

extern "C" {

int astr_decode_graph_create(const astr_paged_args* layers, const astr_new_kv* new_kv, int32_t num_layers,
                             void* workspace, size_t workspace_bytes, void* stream, astr_decode_graph** graph) {
  if (graph == nullptr) return fail(ASTR_ERR_INVALID_ARG, "graph output is NULL");
  *graph = nullptr;
  if (layers == nullptr || num_layers < 1) return fail(ASTR_ERR_INVALID_ARG, "need num_layers >= 1 layer arguments");
  if (stream == nullptr) return fail(ASTR_ERR_INVALID_ARG, "capture needs a non-null stream");
  for (int32_t l = 0; l < num_layers; ++l) {
    const astr_paged_args& a = layers[l];
    if (a.num_splits <= 0)
      return fail(ASTR_ERR_INVALID_ARG, "layer %d: a captured decode needs a fixed plan (num_splits > 0)", l);
    if (a.timing_events != nullptr) return fail(ASTR_ERR_INVALID_ARG, "layer %d: timing_events must be NULL", l);
    if (a.batch != layers[0].batch)
      return fail(ASTR_ERR_INVALID_ARG, "layer %d: batch %d differs from layer 0 (%d); one graph per batch size", l,
                  a.batch, layers[0].batch);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Live run first: validates every layer and loads the kernels before capture.
  int st = enqueue_step(layers, new_kv, num_layers, workspace, workspace_bytes, stream);
  if (st != ASTR_OK) return st;

  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  st = enqueue_step(layers, new_kv, num_layers, workspace, workspace_bytes, stream);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);
  if (st != ASTR_OK) {
    if (g != nullptr) (void)hipGraphDestroy(g);   // cleanup on the error path; its status is not reported
    return st;
  }
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return fail(ASTR_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  astr_decode_graph* out = new (std::nothrow) astr_decode_graph;
  if (out == nullptr) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(g);
    return fail(ASTR_ERR_HIP, "out of host memory");
  }
  out->graph = g;
  out->exec = exec;
  out->num_layers = num_layers;
  out->batch = layers[0].batch;
  *graph = out;
  return ok();
}

int astr_decode_graph_launch(const astr_decode_graph* graph, void* stream) {
  if (graph == nullptr || graph->exec == nullptr) return fail(ASTR_ERR_INVALID_ARG, "graph is NULL");
  const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ASTR_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(e));
  return ok();
}

int astr_decode_graph_destroy(astr_decode_graph* graph) {
  if (graph == nullptr) return ok();
  hipError_t e1 = graph->exec != nullptr ? hipGraphExecDestroy(graph->exec) : hipSuccess;
  hipError_t e2 = graph->graph != nullptr ? hipGraphDestroy(graph->graph) : hipSuccess;
  delete graph;
  if (e1 != hipSuccess) return fail(ASTR_ERR_HIP, "hipGraphExecDestroy: %s", hipGetErrorString(e1));
  if (e2 != hipSuccess) return fail(ASTR_ERR_HIP, "hipGraphDestroy: %s", hipGetErrorString(e2));
  return ok();
}

}  // extern "C"
