// Graph-captured decode steps (include/pa.h, pa_decode_graphs_*): one HIP
// graph per padded batch size holding pa_store_decode (the new tokens' store
// fused into the split kernel and its finalize pass), each step replayed with
// one graph launch (page "nano-vLLM 最小化vLLM重新实现", section 4 "模型运行器":
// decode graphs captured at batch sizes 1, 2, 4, ..., 512; page at
// bxzpzcl.cn/news/2159246, section 3.1).
//
// The graphs hold exactly the kernels an eager pa_store_decode launches, with
// the step's fixed buffers baked in and one more argument: a device count of
// live sequences, which the caller writes with the step's inputs. Rows past it
// are empty contexts inside the kernels, so no padding work runs at launch.
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/pa.h"
#include "launch.h"

struct pa_decode_graphs {
  pa_decode_step step;
  std::vector<int32_t> sizes;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;

  ~pa_decode_graphs() {
    for (hipGraphExec_t e : execs)
      if (e) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs)
      if (g) (void)hipGraphDestroy(g);
  }
};

using pa::fail;
using pa::ok;

extern "C" {

int pa_decode_graphs_create(const pa_decode_step* step, const int32_t* batch_sizes, int32_t count, void* stream,
                            pa_decode_graphs** out) {
  if (!out) return fail(PA_ERR_NULL_POINTER, "out is required");
  *out = nullptr;
  if (!step || !batch_sizes) return fail(PA_ERR_NULL_POINTER, "step and batch_sizes are required");
  if (count <= 0 || count > 32) return fail(PA_ERR_INVALID_ARGUMENT, "count %d outside 1 .. 32", count);
  for (int32_t i = 0; i < count; ++i)
    if (batch_sizes[i] <= 0 || (i > 0 && batch_sizes[i] <= batch_sizes[i - 1]))
      return fail(PA_ERR_INVALID_ARGUMENT, "batch_sizes must be positive and strictly increasing");
  if (!stream) return fail(PA_ERR_INVALID_ARGUMENT, "capture needs a stream other than the legacy default stream");
  if (!step->live_batch || !step->context_lens || !step->k_new || !step->v_new)
    return fail(PA_ERR_NULL_POINTER, "live_batch, context_lens, k_new and v_new are required");
  hipStream_t s = static_cast<hipStream_t>(stream);
  pa_decode_graphs* g = new pa_decode_graphs();
  g->step = *step;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t b = batch_sizes[i];
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      delete g;
      return fail(PA_ERR_HIP, "hipStreamBeginCapture failed for batch %d", b);
    }
    const int st = pa::store_decode_live(g->step, b, s);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &graph);
    if (st != PA_OK || e != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      delete g;
      if (st != PA_OK) return st;  // the captured call's own status and message
      return fail(PA_ERR_HIP, "capture of batch %d failed: %s", b, hipGetErrorString(e));
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    g->graphs.push_back(graph);
    g->execs.push_back(exec);
    g->sizes.push_back(b);
    if (ie != hipSuccess || !exec) {
      delete g;
      return fail(PA_ERR_HIP, "instantiating the batch %d graph failed: %s", b, hipGetErrorString(ie));
    }
  }
  *out = g;
  return ok();
}

int pa_decode_graphs_launch(pa_decode_graphs* g, int32_t batch, void* stream, int32_t* padded) {
  if (!g) return fail(PA_ERR_NULL_POINTER, "graphs are required");
  if (batch <= 0 || batch > g->sizes.back())
    return fail(PA_ERR_INVALID_ARGUMENT, "batch %d outside 1 .. %d", batch, g->sizes.back());
  size_t i = 0;
  while (g->sizes[i] < batch) ++i;
  const int32_t p = g->sizes[i];
  const hipError_t e = hipGraphLaunch(g->execs[i], static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode graph launch: %s", hipGetErrorString(e));
  if (padded) *padded = p;
  return ok();
}

void pa_decode_graphs_destroy(pa_decode_graphs* g) { delete g; }

}  // extern "C"
