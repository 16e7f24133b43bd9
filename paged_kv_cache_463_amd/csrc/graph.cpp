// Step graphs: a fixed sequence of library calls recorded once and replayed
// as one HIP graph launch per step (the role the pages give CUDA graphs in
// the engine's tuning, page "vLLM推理引擎深度实战" §5.3: captured per batch
// size, replayed every decode step).
//
// pa_graph_begin creates a non-blocking stream of default priority and starts
// capturing it; every library call the caller then issues on that stream is
// recorded instead of run; pa_graph_end instantiates the recording. Kernel
// arguments, pointers and grid sizes are frozen in the graph, device memory
// is read at replay time: a graph serves every step whose buffers stay at the
// same addresses and whose batch keeps the same size (lengths and tables may
// change between replays).
#include <new>

#include "pa.h"

#include <hip/hip_runtime.h>

struct pa_graph {
  hipStream_t capture = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  bool capturing = false;
};

extern "C" {

int32_t pa_graph_begin(pa_graph** out, void** capture_stream) {
  if (!out || !capture_stream) return PA_ERR_NULL_PTR;
  *out = nullptr;
  *capture_stream = nullptr;
  pa_graph* g = new (std::nothrow) pa_graph;
  if (!g) return PA_ERR_HIP;
  if (hipStreamCreateWithFlags(&g->capture, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return PA_ERR_HIP;
  }
  if (hipStreamBeginCapture(g->capture, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(g->capture);
    delete g;
    return PA_ERR_HIP;
  }
  g->capturing = true;
  *out = g;
  *capture_stream = g->capture;
  return PA_OK;
}

int32_t pa_graph_end(pa_graph* g) {
  if (!g) return PA_ERR_NULL_PTR;
  if (!g->capturing) return PA_ERR_SHAPE;
  g->capturing = false;
  if (hipStreamEndCapture(g->capture, &g->graph) != hipSuccess || !g->graph) return PA_ERR_HIP;
  if (hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0) != hipSuccess) {
    g->exec = nullptr;
    return PA_ERR_HIP;
  }
  return PA_OK;
}

int32_t pa_graph_launch(pa_graph* g, void* stream) {
  if (!g) return PA_ERR_NULL_PTR;
  if (!g->exec) return PA_ERR_SHAPE;
  return hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

void pa_graph_destroy(pa_graph* g) {
  if (!g) return;
  if (g->capturing) {                        // abandon an unfinished recording
    hipGraph_t partial = nullptr;
    if (hipStreamEndCapture(g->capture, &partial) == hipSuccess && partial) (void)hipGraphDestroy(partial);
    (void)hipGetLastError();
  }
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->capture) (void)hipStreamDestroy(g->capture);
  delete g;
}

}  // extern "C"
