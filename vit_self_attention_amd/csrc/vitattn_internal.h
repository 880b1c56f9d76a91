// Internal interface between the C-ABI entry points (vitattn_api.cpp), the
// host-only argument checks (vitattn_host.cpp) and the gfx950 kernels
// (vitattn_fwd.hip, vitattn_linear.hip).  Not installed; not part of the ABI.
#pragma once

#include <stdint.h>

namespace vitattn {

// Per-launch description of one attention problem.  Strides are in 16-bit
// elements.  For (image b, head h, token n) the row of Q starts at
// q + b*q_sb + h*q_sh + n*q_st, and likewise for k, v and out.
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st;
  int B, H, N, D;
  float scale;
  bool f16;  // elements are fp16 (true) or bf16 (false): inputs, probabilities, output
};

// Checks the arguments of one vitattn_fwd call and fills `a`.  Returns
// VITATTN_OK (with *empty set for a problem with nothing to compute) or a
// negative VITATTN_ERR_* code; host only, no HIP call.
int check_fwd(const void* qkv_or_q, const void* k, const void* v, void* out, int B, int H, int N,
              int D, float scale, int layout, FwdArgs* a, bool* empty);

// The size limits of vitattn_fwd for a non-empty problem with valid sizes
// (B, H, N >= 1, D 64 or 72; layout without the format flag): VITATTN_OK or
// VITATTN_ERR_TOO_LARGE.  Host only.
int check_fwd_limits(int B, int H, int N, int D, int layout);

// How the attention kernel is launched for a problem.  A work item is one
// (image, head, block of queries); each wave owns 32 queries of it.
struct FwdShape {
  int waves;    // waves per workgroup: 1, 2 or 4
  bool split;   // the four waves split the keys of one 32-query block
  int qblocks;  // query blocks per (image, head)
  int items;    // B * H * qblocks
  int grid;     // workgroups: one per item, or fewer that loop over the items
};

// Launch shape on a part with `compute_units` compute units (0 if unknown:
// then no workgroup loops).  Host only.
FwdShape fwd_shape(int B, int H, int N, int compute_units);

// Enqueues the forward kernel on `stream` (a hipStream_t).  Arguments are
// already validated.  Returns 0 or a negative VITATTN_ERR_* code.
int launch_fwd(const FwdArgs& a, void* stream);

// Compute units of the current device (0 if unknown), cached per device.
int compute_units();

// One linear layer: out[m][n] = sum_k x[m][k] * w[n][k] + bias[n]
// (+ residual[m][n]); x [M][K], w [Nout][K], bias [Nout], residual and out
// [M][Nout], all 16-bit.  Arguments are already validated (K a multiple of
// 32, Nout a multiple of 8, byte offsets below 2^32).
struct LinearCall {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* bias;      // NULL: no bias
  const uint16_t* residual;  // NULL: no residual
  uint16_t* out;
  int M, K, Nout;
  bool f16;
};

// Checks the arguments of one vitattn_linear call and fills `c`, as
// check_fwd does.
int check_linear(const void* x, const void* w, const void* bias, const void* residual, void* out,
                 int M, int K, int Nout, int flags, LinearCall* c, bool* empty);

// Enqueues the linear kernel on `stream`.  Returns 0 or VITATTN_ERR_LAUNCH.
int launch_linear(const LinearCall& c, void* stream);

}  // namespace vitattn
