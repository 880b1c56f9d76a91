// C-ABI entry points of libvitattn: argument validation on the host
// (vitattn_host.cpp), then one kernel launch (vitattn_fwd, vitattn_linear)
// or a HIP graph of such launches (plans).  Every check runs before any HIP
// call, so a bad argument never reaches the device.
#include "vitattn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "vitattn_internal.h"

extern "C" int vitattn_fwd(const void* qkv_or_q, const void* k, const void* v, void* out,
                           int B, int H, int N, int D, float scale, int layout, void* stream) {
  vitattn::FwdArgs a;
  bool empty;
  const int st = vitattn::check_fwd(qkv_or_q, k, v, out, B, H, N, D, scale, layout, &a, &empty);
  if (st != VITATTN_OK || empty) return st;
  return vitattn::launch_fwd(a, stream);
}

extern "C" int vitattn_fwd_shape(int B, int H, int N, int D, int layout, int* waves, int* split_keys,
                                 int* items, int* workgroups) {
  if (!waves || !split_keys || !items || !workgroups) return VITATTN_ERR_NULL_POINTER;
  if ((layout & ~VITATTN_DTYPE_FP16) != VITATTN_LAYOUT_SEPARATE_BHND &&
      (layout & ~VITATTN_DTYPE_FP16) != VITATTN_LAYOUT_PACKED_BN3HD)
    return VITATTN_ERR_BAD_LAYOUT;
  if (B < 0 || H < 0 || N < 0) return VITATTN_ERR_BAD_SIZE;
  if (D != 64 && D != 72) return VITATTN_ERR_UNSUPPORTED_D;
  {
    const int st = vitattn::check_fwd_limits(B, H, N, D, layout & ~VITATTN_DTYPE_FP16);
    if (st != VITATTN_OK) return st;
  }
  const vitattn::FwdShape s = vitattn::fwd_shape(B, H, N, vitattn::compute_units());
  *waves = s.waves;
  *split_keys = s.split ? 1 : 0;
  *items = s.items;
  *workgroups = s.grid;
  return VITATTN_OK;
}

// A recorded sequence of forward calls: one executable HIP graph, bound to
// the device that was current when it was recorded.
struct vitattn_plan_s {
  hipGraphExec_t exec = nullptr;  // NULL when every recorded call was empty
};

extern "C" int vitattn_plan_create(vitattn_plan* plan, int layers, const void* const* qkv_or_q,
                                   const void* const* k, const void* const* v, void* const* out,
                                   int B, int H, int N, int D, float scale, int layout) {
  if (!plan) return VITATTN_ERR_NULL_POINTER;
  *plan = nullptr;
  if (layers < 1) return VITATTN_ERR_BAD_SIZE;
  if (!qkv_or_q || !out) return VITATTN_ERR_NULL_POINTER;
  const bool separate = (layout & ~VITATTN_DTYPE_FP16) == VITATTN_LAYOUT_SEPARATE_BHND;
  if (separate && (!k || !v)) return VITATTN_ERR_NULL_POINTER;
  if (!separate && (k || v)) return VITATTN_ERR_BAD_LAYOUT;
  // every call is checked before anything is recorded
  std::vector<vitattn::FwdArgs> calls;
  calls.reserve(layers);
  for (int l = 0; l < layers; ++l) {
    vitattn::FwdArgs a;
    bool empty;
    const int st = vitattn::check_fwd(qkv_or_q[l], separate ? k[l] : nullptr, separate ? v[l] : nullptr,
                                      out[l], B, H, N, D, scale, layout, &a, &empty);
    if (st != VITATTN_OK) return st;
    if (!empty) calls.push_back(a);
  }
  vitattn_plan_s* p = new (std::nothrow) vitattn_plan_s;
  if (!p) return VITATTN_ERR_GRAPH;
  if (calls.empty()) {
    *plan = p;
    return VITATTN_OK;
  }
  // record the calls on a private stream (default priority), in order
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    delete p;
    return VITATTN_ERR_GRAPH;
  }
  int status = VITATTN_OK;
  hipGraph_t graph = nullptr;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed) != hipSuccess) {
    status = VITATTN_ERR_GRAPH;
  } else {
    for (const vitattn::FwdArgs& a : calls) {
      if (vitattn::launch_fwd(a, s) != VITATTN_OK) {
        status = VITATTN_ERR_GRAPH;
        break;
      }
    }
    // the capture is always ended, also after a failed launch
    if (hipStreamEndCapture(s, &graph) != hipSuccess || !graph) status = VITATTN_ERR_GRAPH;
  }
  if (status == VITATTN_OK && hipGraphInstantiate(&p->exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    p->exec = nullptr;
    status = VITATTN_ERR_GRAPH;
  }
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(s);
  if (status != VITATTN_OK) {
    delete p;
    return status;
  }
  *plan = p;
  return VITATTN_OK;
}

extern "C" int vitattn_plan_launch(vitattn_plan plan, void* stream) {
  if (!plan) return VITATTN_ERR_NULL_POINTER;
  if (!plan->exec) return VITATTN_OK;
  return hipGraphLaunch(plan->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? VITATTN_OK
                                                                                  : VITATTN_ERR_GRAPH;
}

extern "C" int vitattn_plan_destroy(vitattn_plan plan) {
  if (!plan) return VITATTN_OK;
  const bool ok = !plan->exec || hipGraphExecDestroy(plan->exec) == hipSuccess;
  delete plan;
  return ok ? VITATTN_OK : VITATTN_ERR_GRAPH;
}

extern "C" int vitattn_linear(const void* x, const void* w, const void* bias, const void* residual,
                              void* out, int M, int K, int Nout, int flags, void* stream) {
  vitattn::LinearCall c;
  bool empty;
  const int st = vitattn::check_linear(x, w, bias, residual, out, M, K, Nout, flags, &c, &empty);
  if (st != VITATTN_OK || empty) return st;
  return vitattn::launch_linear(c, stream) == 0 ? VITATTN_OK : VITATTN_ERR_LAUNCH;
}
