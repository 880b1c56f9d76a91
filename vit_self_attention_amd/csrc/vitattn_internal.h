// Internal interface between the C-ABI entry points (vitattn_api.cpp) and
// the gfx950 kernels (vitattn_fwd.hip).  Not installed; not part of the ABI.
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

// Enqueues the forward kernel on `stream` (a hipStream_t).  Arguments are
// already validated.  Returns 0 or a negative VITATTN_ERR_* code.
int launch_fwd(const FwdArgs& a, void* stream);

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

// Enqueues the linear kernel on `stream`.  Returns 0 or VITATTN_ERR_LAUNCH.
int launch_linear(const LinearCall& c, void* stream);

// Number of waves per workgroup the launcher picks for a problem (1, 2 or 4);
// exposed for tests and the benchmark's reporting.
int pick_waves(int B, int H, int N);

}  // namespace vitattn
