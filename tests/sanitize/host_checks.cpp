// Drives the host-only argument checks of libvitattn (vitattn_host.cpp)
// through every error path and the size limits, for a build with address
// and undefined-behaviour sanitizers.  Prints one line per case:
//   <case> <status> [<launch shape>]
// which tests/test_sanitize.py compares with the codes include/vitattn.h
// documents.  Pointers are fake addresses that are never dereferenced.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "vitattn.h"
#include "vitattn_internal.h"

namespace {

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

const uintptr_t kIn = uintptr_t(1) << 44, kOut = uintptr_t(1) << 45;

void fwd(const char* name, const void* q, const void* k, const void* v, void* o, int B, int H, int N,
         int D, float scale, int layout) {
  vitattn::FwdArgs a;
  bool empty = false;
  const int st = vitattn::check_fwd(q, k, v, o, B, H, N, D, scale, layout, &a, &empty);
  printf("%s %d%s\n", name, st, empty ? " empty" : "");
}

void lin(const char* name, const void* x, const void* w, const void* b, const void* r, void* o, int M,
         int K, int Nout, int flags) {
  vitattn::LinearCall c;
  bool empty = false;
  const int st = vitattn::check_linear(x, w, b, r, o, M, K, Nout, flags, &c, &empty);
  printf("%s %d%s\n", name, st, empty ? " empty" : "");
}

void shape(const char* name, int B, int H, int N, int cus) {
  const vitattn::FwdShape s = vitattn::fwd_shape(B, H, N, cus);
  printf("%s 0 waves=%d split=%d qblocks=%d items=%d grid=%d\n", name, s.waves, s.split ? 1 : 0,
         s.qblocks, s.items, s.grid);
}

}  // namespace

int main() {
  const int PK = VITATTN_LAYOUT_PACKED_BN3HD, SP = VITATTN_LAYOUT_SEPARATE_BHND;
  // valid calls
  fwd("fwd_ok_packed", P(kIn), nullptr, nullptr, P(kOut), 48, 16, 729, 72, 0.1178f, PK);
  fwd("fwd_ok_separate", P(kIn), P(kIn + (1 << 28)), P(kIn + (2 << 28)), P(kOut), 1, 12, 197, 64, 0.125f, SP);
  fwd("fwd_ok_fp16", P(kIn), nullptr, nullptr, P(kOut), 2, 16, 256, 72, 0.1f, PK | VITATTN_DTYPE_FP16);
  fwd("fwd_ok_zero_scale", P(kIn), nullptr, nullptr, P(kOut), 1, 1, 1, 64, 0.0f, PK);
  fwd("fwd_empty_b", nullptr, nullptr, nullptr, nullptr, 0, 16, 729, 72, 0.1f, PK);
  fwd("fwd_empty_n", nullptr, nullptr, nullptr, nullptr, 4, 16, 0, 64, 0.1f, SP);
  // each error on its own
  fwd("fwd_bad_layout", P(kIn), nullptr, nullptr, P(kOut), 1, 1, 8, 64, 0.1f, 7);
  fwd("fwd_packed_with_k", P(kIn), P(kIn), nullptr, P(kOut), 1, 1, 8, 64, 0.1f, PK);
  fwd("fwd_negative_b", P(kIn), nullptr, nullptr, P(kOut), -1, 1, 8, 64, 0.1f, PK);
  fwd("fwd_negative_n", P(kIn), nullptr, nullptr, P(kOut), 1, 1, INT_MIN, 64, 0.1f, PK);
  fwd("fwd_d80", P(kIn), nullptr, nullptr, P(kOut), 1, 1, 8, 80, 0.1f, PK);
  fwd("fwd_nan_scale", P(kIn), nullptr, nullptr, P(kOut), 1, 1, 8, 64, NAN, PK);
  fwd("fwd_inf_scale", P(kIn), nullptr, nullptr, P(kOut), 1, 1, 8, 64, -INFINITY, PK);
  fwd("fwd_null_out", P(kIn), nullptr, nullptr, nullptr, 1, 1, 8, 64, 0.1f, PK);
  fwd("fwd_null_v", P(kIn), P(kIn + 4096), nullptr, P(kOut), 1, 1, 8, 64, 0.1f, SP);
  fwd("fwd_misaligned_q", P(kIn + 8), nullptr, nullptr, P(kOut), 1, 1, 8, 64, 0.1f, PK);
  fwd("fwd_misaligned_k", P(kIn), P(kIn + 4104), P(kIn + 8192), P(kOut), 1, 1, 8, 64, 0.1f, SP);
  fwd("fwd_overlap_packed", P(kIn), nullptr, nullptr, P(kIn + 4096), 1, 1, 64, 64, 0.1f, PK);
  fwd("fwd_overlap_separate_v", P(kIn), P(kIn + (1 << 20)), P(kOut + 1024), P(kOut), 1, 1, 64, 64, 0.1f, SP);
  fwd("fwd_adjacent_no_overlap", P(kIn), nullptr, nullptr, P(kIn + 3 * 64 * 64 * 2), 1, 1, 64, 64, 0.1f, PK);
  // size limits, each product near the edge of int64 without overflowing
  fwd("fwd_huge_all", P(kIn), nullptr, nullptr, P(kOut), INT_MAX, INT_MAX, INT_MAX, 64, 0.1f, PK);
  fwd("fwd_huge_bh", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), INT_MAX, INT_MAX, 1, 64, 0.1f, SP);
  fwd("fwd_huge_n", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), 1, 1, INT_MAX, 64, 0.1f, SP);
  fwd("fwd_n_limit", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), 1, 1, 1 << 24, 64, 0.1f, SP);
  fwd("fwd_n_past_limit", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), 1, 1, (1 << 24) + 1, 64, 0.1f, SP);
  fwd("fwd_rows_past_2_40", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), 1 << 20, 1 << 10, 1 << 11, 64, 0.1f, SP);
  fwd("fwd_token_stride", P(kIn), nullptr, nullptr, P(kOut), 1, 1 << 17, 1, 72, 0.1f, PK);
  fwd("fwd_items_past_2_30", P(kIn), P(kIn + (uintptr_t(1) << 42)), P(kIn + (uintptr_t(2) << 42)), P(kOut), 1 << 16, 1 << 10, 2048, 64, 0.1f, SP);
  // linear layers
  lin("lin_ok", P(kIn), P(kIn + (1 << 30)), P(kIn + (2u << 30)), nullptr, P(kOut), 34992, 1152, 3456, 0);
  lin("lin_ok_inplace_residual", P(kIn), P(kIn + (1 << 30)), nullptr, P(kOut), P(kOut), 512, 1152, 1152, 0);
  lin("lin_empty", nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1152, 1152, 0);
  lin("lin_bad_flags", P(kIn), P(kIn), nullptr, nullptr, P(kOut), 8, 32, 8, 3);
  lin("lin_negative_m", P(kIn), P(kIn), nullptr, nullptr, P(kOut), -8, 32, 8, 0);
  lin("lin_k_not_32", P(kIn), P(kIn), nullptr, nullptr, P(kOut), 8, 48, 8, 0);
  lin("lin_nout_not_8", P(kIn), P(kIn), nullptr, nullptr, P(kOut), 8, 32, 12, 0);
  lin("lin_null_w", P(kIn), nullptr, nullptr, nullptr, P(kOut), 8, 32, 8, 0);
  lin("lin_misaligned_bias", P(kIn), P(kIn + 4096), P(kIn + 8200), nullptr, P(kOut), 8, 32, 8, 0);
  lin("lin_x_4gib", P(kIn), P(kIn), nullptr, nullptr, P(kOut), 1 << 21, 1024, 8, 0);
  lin("lin_huge_all", P(kIn), P(kIn), nullptr, nullptr, P(kOut), INT_MAX, INT_MAX & ~31, INT_MAX & ~7, 0);
  lin("lin_overlap_x", P(kIn), P(kOut + (1 << 24)), nullptr, nullptr, P(kIn + 64), 8, 32, 8, 0);
  lin("lin_shifted_residual", P(kIn), P(kIn + 4096), nullptr, P(kOut + 16), P(kOut), 8, 32, 8, 0);
  // launch shapes
  shape("shape_c1", 1, 12, 197, 256);
  shape("shape_c3", 2, 16, 256, 256);
  shape("shape_c4", 24, 16, 257, 256);
  shape("shape_c5", 48, 16, 729, 256);
  shape("shape_c5_no_device", 48, 16, 729, 0);
  shape("shape_384x6", 6, 16, 729, 256);    // 1.125 items per slot: loops
  shape("shape_384x9", 9, 16, 729, 256);    // 1.6875 items per slot: loops
  shape("shape_n1024x4", 4, 16, 1024, 256); // one item per slot: one workgroup each
  shape("shape_one_token", 1, 1, 1, 256);
  shape("shape_max_n", 1, 1, 1 << 24, 256);
  // status strings: every code has one, unknown codes a fixed text
  for (int code = 0; code >= -12; --code) printf("strerror_%d %s\n", -code, vitattn_strerror(code));
  printf("version %d\n", vitattn_version());
  return 0;
}
