// C-ABI entry points of libvitattn: argument validation on the host, then
// one kernel launch (vitattn_fwd) or a HIP graph of such launches (plans).
// Every check runs before any HIP call, so a bad argument never reaches the
// device.
#include "vitattn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "vitattn_internal.h"

namespace {

constexpr int kVersion = 10000 * 0 + 100 * 1 + 0;  // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

// Checks the arguments of one forward call and fills `a`.  Returns
// VITATTN_OK with *empty set for a problem with nothing to compute, or a
// negative code; makes no HIP call.
int prepare(const void* qkv_or_q, const void* k, const void* v, void* out, int B, int H, int N,
            int D, float scale, int layout, vitattn::FwdArgs* a, bool* empty) {
  *empty = false;
  const bool f16 = (layout & VITATTN_DTYPE_FP16) != 0;
  layout &= ~VITATTN_DTYPE_FP16;
  if (layout != VITATTN_LAYOUT_SEPARATE_BHND && layout != VITATTN_LAYOUT_PACKED_BN3HD)
    return VITATTN_ERR_BAD_LAYOUT;
  if (layout == VITATTN_LAYOUT_PACKED_BN3HD && (k != nullptr || v != nullptr))
    return VITATTN_ERR_BAD_LAYOUT;
  if (B < 0 || H < 0 || N < 0) return VITATTN_ERR_BAD_SIZE;
  if (D != 64 && D != 72) return VITATTN_ERR_UNSUPPORTED_D;
  if (!isfinite(scale)) return VITATTN_ERR_BAD_SCALE;
  // An empty problem has nothing to read or write; its buffers may be NULL
  // (a zero-element tensor usually has no storage).
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return VITATTN_OK;
  }
  if (!qkv_or_q || !out) return VITATTN_ERR_NULL_POINTER;
  if (layout == VITATTN_LAYOUT_SEPARATE_BHND && (!k || !v)) return VITATTN_ERR_NULL_POINTER;
  if (!aligned16(qkv_or_q) || !aligned16(out)) return VITATTN_ERR_MISALIGNED;
  if (layout == VITATTN_LAYOUT_SEPARATE_BHND && (!aligned16(k) || !aligned16(v)))
    return VITATTN_ERR_MISALIGNED;

  // Problem-size limits: element offsets are 64-bit inside the kernel; the
  // grid is one workgroup per (image, head, query block) and must fit int32.
  const int64_t rows = static_cast<int64_t>(B) * H * N;  // (b, h, token) rows
  if (rows > (int64_t(1) << 40)) return VITATTN_ERR_TOO_LARGE;
  const int64_t pairs = static_cast<int64_t>(B) * H;
  // a key tile (64 token rows) must span less than 2 GiB: the kernel
  // addresses its rows with 32-bit byte offsets
  const int64_t token_stride = layout == VITATTN_LAYOUT_PACKED_BN3HD ? 3 * static_cast<int64_t>(H) * D : D;
  if (64 * token_stride * 2 >= (int64_t(1) << 31)) return VITATTN_ERR_TOO_LARGE;
  if (pairs * ((static_cast<int64_t>(N) + 31) / 32) > (int64_t(1) << 30))
    return VITATTN_ERR_TOO_LARGE;

  const int64_t t_bytes = rows * D * 2;  // one of Q, K, V or O, in bytes
  if (layout == VITATTN_LAYOUT_PACKED_BN3HD) {
    if (overlaps(out, t_bytes, qkv_or_q, 3 * t_bytes)) return VITATTN_ERR_OVERLAP;
  } else {
    if (overlaps(out, t_bytes, qkv_or_q, t_bytes) || overlaps(out, t_bytes, k, t_bytes) ||
        overlaps(out, t_bytes, v, t_bytes))
      return VITATTN_ERR_OVERLAP;
  }

  *a = vitattn::FwdArgs{};
  a->B = B;
  a->H = H;
  a->N = N;
  a->D = D;
  a->scale = scale;
  a->f16 = f16;
  a->o = static_cast<uint16_t*>(out);
  const int64_t hd = static_cast<int64_t>(H) * D;
  if (layout == VITATTN_LAYOUT_PACKED_BN3HD) {
    const uint16_t* base = static_cast<const uint16_t*>(qkv_or_q);
    a->q = base;
    a->k = base + hd;
    a->v = base + 2 * hd;
    const int64_t st = 3 * hd, sb = static_cast<int64_t>(N) * st;
    a->q_sb = a->k_sb = a->v_sb = sb;
    a->q_sh = a->k_sh = a->v_sh = D;
    a->q_st = a->k_st = a->v_st = st;
    a->o_sb = static_cast<int64_t>(N) * hd;
    a->o_sh = D;
    a->o_st = hd;
  } else {
    a->q = static_cast<const uint16_t*>(qkv_or_q);
    a->k = static_cast<const uint16_t*>(k);
    a->v = static_cast<const uint16_t*>(v);
    const int64_t sh = static_cast<int64_t>(N) * D, sb = static_cast<int64_t>(H) * sh;
    a->q_sb = a->k_sb = a->v_sb = a->o_sb = sb;
    a->q_sh = a->k_sh = a->v_sh = a->o_sh = sh;
    a->q_st = a->k_st = a->v_st = a->o_st = D;
  }
  return VITATTN_OK;
}

}  // namespace

extern "C" int vitattn_fwd(const void* qkv_or_q, const void* k, const void* v, void* out,
                           int B, int H, int N, int D, float scale, int layout, void* stream) {
  vitattn::FwdArgs a;
  bool empty;
  const int st = prepare(qkv_or_q, k, v, out, B, H, N, D, scale, layout, &a, &empty);
  if (st != VITATTN_OK || empty) return st;
  return vitattn::launch_fwd(a, stream);
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
    const int st = prepare(qkv_or_q[l], separate ? k[l] : nullptr, separate ? v[l] : nullptr, out[l],
                           B, H, N, D, scale, layout, &a, &empty);
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
  if ((flags & ~VITATTN_DTYPE_FP16) != 0) return VITATTN_ERR_BAD_LAYOUT;
  if (M < 0 || K < 0 || Nout < 0) return VITATTN_ERR_BAD_SIZE;
  if (K == 0 || K % 32 != 0 || Nout % 8 != 0) return VITATTN_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || Nout == 0) return VITATTN_OK;
  if (!x || !w || !out) return VITATTN_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (bias && !aligned16(bias)) ||
      (residual && !aligned16(residual)))
    return VITATTN_ERR_MISALIGNED;
  // the kernel addresses x and w rows with 32-bit byte offsets
  const int64_t x_bytes = static_cast<int64_t>(M) * K * 2, w_bytes = static_cast<int64_t>(Nout) * K * 2;
  if (x_bytes >= (int64_t(1) << 32) || w_bytes >= (int64_t(1) << 32)) return VITATTN_ERR_TOO_LARGE;
  const int64_t o_bytes = static_cast<int64_t>(M) * Nout * 2;
  if (o_bytes >= (int64_t(1) << 40)) return VITATTN_ERR_TOO_LARGE;
  if (overlaps(out, o_bytes, x, x_bytes) || overlaps(out, o_bytes, w, w_bytes) ||
      overlaps(out, o_bytes, bias, static_cast<int64_t>(Nout) * 2))
    return VITATTN_ERR_OVERLAP;
  // the residual may be the output itself (an in-place residual add: every
  // element is read and written by the same lane), but not a shifted view
  if (residual && residual != out && overlaps(out, o_bytes, residual, o_bytes)) return VITATTN_ERR_OVERLAP;
  vitattn::LinearCall c{};
  c.x = static_cast<const uint16_t*>(x);
  c.w = static_cast<const uint16_t*>(w);
  c.bias = static_cast<const uint16_t*>(bias);
  c.residual = static_cast<const uint16_t*>(residual);
  c.out = static_cast<uint16_t*>(out);
  c.M = M;
  c.K = K;
  c.Nout = Nout;
  c.f16 = (flags & VITATTN_DTYPE_FP16) != 0;
  return vitattn::launch_linear(c, stream) == 0 ? VITATTN_OK : VITATTN_ERR_LAUNCH;
}

extern "C" const char* vitattn_strerror(int status) {
  switch (status) {
    case VITATTN_OK: return "success";
    case VITATTN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case VITATTN_ERR_BAD_SIZE: return "B, H or N is negative";
    case VITATTN_ERR_UNSUPPORTED_D: return "head dimension D must be 64 or 72";
    case VITATTN_ERR_BAD_SCALE: return "scale must be finite";
    case VITATTN_ERR_BAD_LAYOUT:
      return "unknown layout, or k/v passed with the packed layout";
    case VITATTN_ERR_MISALIGNED: return "device pointers must be 16-byte aligned";
    case VITATTN_ERR_TOO_LARGE: return "problem exceeds the launch limits";
    case VITATTN_ERR_LAUNCH: return "kernel launch failed";
    case VITATTN_ERR_OVERLAP: return "out overlaps an input buffer";
    case VITATTN_ERR_GRAPH: return "recording or launching the HIP graph failed";
    case VITATTN_ERR_UNSUPPORTED_SHAPE:
      return "linear layer: K must be a positive multiple of 32 and Nout a multiple of 8";
    default: return "unknown status";
  }
}

extern "C" int vitattn_version(void) { return kVersion; }
