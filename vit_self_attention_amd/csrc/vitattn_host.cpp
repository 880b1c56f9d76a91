// Host-only part of libvitattn: argument checking for every entry point and
// the launch shape of the attention kernel.  Plain C++ with no HIP header,
// so that it builds with the host compiler alone (the CPU tests build it
// with address and undefined-behaviour sanitizers and drive every check).
//
// The checks follow the boundary the Pi0 Flash Attention tutorial sets for
// the swapped-in attention (section 3.2: the block's fused qkv activation
// in, the same output as before; section 5.2: a mismatched argument is an
// error, not a silent fallback): every argument is checked before any device
// work and a failed check returns its negative status code.
#include <math.h>
#include <stdint.h>

#include "vitattn.h"
#include "vitattn_internal.h"

namespace vitattn {

namespace {

constexpr int kVersion = 10000 * 0 + 100 * 2 + 0;  // 0.2.0
constexpr int kMaxTokens = 1 << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + a_bytes) and [b, b + b_bytes) share a byte
bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  if (!a || !b || a_bytes <= 0 || b_bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(b_bytes) && b0 < a0 + static_cast<uintptr_t>(a_bytes);
}

}  // namespace

int check_fwd_limits(int B, int H, int N, int D, int layout) {
  if (B <= 0 || H <= 0 || N <= 0) return VITATTN_OK;  // empty, or rejected earlier
  // Element offsets are 64-bit in the kernel, and the (b, h, token) rows
  // number at most 2^40 (every product below then stays far inside int64;
  // B*H is formed first, below 2^62, and compared before it meets N).
  // The kernel's token arithmetic is 32-bit: N stays far below 2^31.
  if (N > kMaxTokens) return VITATTN_ERR_TOO_LARGE;
  const int64_t pairs = static_cast<int64_t>(B) * H;
  if (pairs > (int64_t(1) << 40) / N) return VITATTN_ERR_TOO_LARGE;
  // A key tile (64 token rows) must span less than 2 GiB: the kernel
  // addresses its rows with 32-bit byte offsets.
  const int64_t token_stride =
      layout == VITATTN_LAYOUT_PACKED_BN3HD ? 3 * static_cast<int64_t>(H) * D : D;
  if (64 * token_stride * 2 >= (int64_t(1) << 31)) return VITATTN_ERR_TOO_LARGE;
  // the work items, one per (image, head, block of 32 queries), must fit a
  // 32-bit count
  if (pairs * ((static_cast<int64_t>(N) + 31) / 32) > (int64_t(1) << 30)) return VITATTN_ERR_TOO_LARGE;
  return VITATTN_OK;
}

int check_fwd(const void* qkv_or_q, const void* k, const void* v, void* out, int B, int H, int N,
              int D, float scale, int layout, FwdArgs* a, bool* empty) {
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

  {
    const int st = check_fwd_limits(B, H, N, D, layout);
    if (st != VITATTN_OK) return st;
  }
  const int64_t rows = static_cast<int64_t>(B) * H * N;  // (b, h, token) rows, at most 2^40
  const int64_t t_bytes = rows * D * 2;  // one of Q, K, V or O, in bytes
  if (layout == VITATTN_LAYOUT_PACKED_BN3HD) {
    if (overlaps(out, t_bytes, qkv_or_q, 3 * t_bytes)) return VITATTN_ERR_OVERLAP;
  } else {
    if (overlaps(out, t_bytes, qkv_or_q, t_bytes) || overlaps(out, t_bytes, k, t_bytes) ||
        overlaps(out, t_bytes, v, t_bytes))
      return VITATTN_ERR_OVERLAP;
  }

  *a = FwdArgs{};
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

int check_linear(const void* x, const void* w, const void* bias, const void* residual, void* out,
                 int M, int K, int Nout, int flags, LinearCall* c, bool* empty) {
  *empty = false;
  if ((flags & ~VITATTN_DTYPE_FP16) != 0) return VITATTN_ERR_BAD_LAYOUT;
  if (M < 0 || K < 0 || Nout < 0) return VITATTN_ERR_BAD_SIZE;
  if (K == 0 || K % 32 != 0 || Nout % 8 != 0) return VITATTN_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || Nout == 0) {
    *empty = true;
    return VITATTN_OK;
  }
  if (!x || !w || !out) return VITATTN_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (bias && !aligned16(bias)) ||
      (residual && !aligned16(residual)))
    return VITATTN_ERR_MISALIGNED;
  // The kernel addresses x and w rows with 32-bit byte offsets.  Element
  // counts are products of two ints (below 2^62) and are compared before
  // they are turned into bytes.
  const int64_t x_elems = static_cast<int64_t>(M) * K, w_elems = static_cast<int64_t>(Nout) * K;
  if (x_elems >= (int64_t(1) << 31) || w_elems >= (int64_t(1) << 31)) return VITATTN_ERR_TOO_LARGE;
  const int64_t o_elems = static_cast<int64_t>(M) * Nout;
  if (o_elems >= (int64_t(1) << 39)) return VITATTN_ERR_TOO_LARGE;
  const int64_t x_bytes = 2 * x_elems, w_bytes = 2 * w_elems, o_bytes = 2 * o_elems;
  if (overlaps(out, o_bytes, x, x_bytes) || overlaps(out, o_bytes, w, w_bytes) ||
      overlaps(out, o_bytes, bias, static_cast<int64_t>(Nout) * 2))
    return VITATTN_ERR_OVERLAP;
  // the residual may be the output itself (an in-place residual add: every
  // element is read and written by the same lane), but not a shifted view
  if (residual && residual != out && overlaps(out, o_bytes, residual, o_bytes)) return VITATTN_ERR_OVERLAP;
  *c = LinearCall{};
  c->x = static_cast<const uint16_t*>(x);
  c->w = static_cast<const uint16_t*>(w);
  c->bias = static_cast<const uint16_t*>(bias);
  c->residual = static_cast<const uint16_t*>(residual);
  c->out = static_cast<uint16_t*>(out);
  c->M = M;
  c->K = K;
  c->Nout = Nout;
  c->f16 = (flags & VITATTN_DTYPE_FP16) != 0;
  return VITATTN_OK;
}

FwdShape fwd_shape(int B, int H, int N, int compute_units) {
  FwdShape s{};
  const int64_t pairs = static_cast<int64_t>(B) * H;
  const int64_t ntiles = (static_cast<int64_t>(N) + 63) / 64;
  // (256, the MI355X's count, when the device is unknown)
  const int64_t cus = compute_units > 0 ? compute_units : 256;
  // Split keys: the four waves of a workgroup share one 32-query block and
  // take its key tiles in turn (w, w + 4, ...), for four times the
  // workgroups of 128-query items.  For short sequences (2..4 key tiles)
  // while those items would not give every compute unit one: with a
  // workgroup per compute unit or more the 128-query items win (8 images
  // at N = 256: 9.2 against 10.2 us split; 12 at N = 200: 11.8 against
  // 13.4; below, 4 images at N = 256: 6.0 split against 8.5).  For longer
  // ones while four-wave items would not reach half the compute units
  // (where one- and two-wave workgroups ran before: SigLIP 384 px, one
  // image, 10.4 against 13.1 us; ViT-B/16 384 px, one image, 6.1 against
  // 10.2; one head at N = 2048, 11.4 against 24.7).  Within the bounds of
  // the kernel's multiply-shift coordinate arithmetic (fewer than 2048
  // items, items * qblocks <= 2^16, pairs * H <= 2^20).
  const int64_t qb32 = (static_cast<int64_t>(N) + 31) / 32, qb128 = (static_cast<int64_t>(N) + 127) / 128;
  const bool div_ok = qb32 <= 255 && H <= 2047 && pairs * qb32 < 2048 &&
                      pairs * qb32 * qb32 <= (int64_t(1) << 16) && pairs * H <= (int64_t(1) << 20);
  if (ntiles >= 2 && div_ok && (ntiles <= 4 ? pairs * qb128 < cus : pairs * qb128 < cus / 2)) {
    s.waves = 4;
    s.split = true;
    s.qblocks = static_cast<int>(qb32);
  } else {
    // Otherwise the largest workgroup that still gives a workgroup to at
    // least half the compute units.
    // Every workgroup holds a whole LDS ring, so two fit on a compute unit
    // whatever their size: four waves share each fetched K/V tile four
    // ways, and two or one leave a compute unit with four or two waves to
    // hide latency with.  On 256 compute units (A/B, us per call, against
    // the earlier rule of at least 512 workgroups): 384 px x 2, 4 and 5
    // images 14.1, 21.5 and 23.5 against 25.8, 28.2 and 30.0; ViT-L/14 at
    // 4, 6, 8 and 10 images 7.9, 10.4, 10.6 and 10.9 against 13.6, 14.4,
    // 15.0 and 15.4; one image at N = 1025 15.9 against 29.6.  Below half,
    // more and smaller workgroups spread the latency better.
    const int64_t min_wgs = cus / 2;
    s.waves = 1;
    for (int nw = 4; nw > 1; nw >>= 1) {
      const int64_t qb = (static_cast<int64_t>(N) + 32 * nw - 1) / (32 * nw);
      if (pairs * qb >= min_wgs) {
        s.waves = nw;
        break;
      }
    }
    s.qblocks = static_cast<int>((static_cast<int64_t>(N) + 32 * s.waves - 1) / (32 * s.waves));
  }
  s.items = static_cast<int>(pairs * s.qblocks);
  s.grid = s.items;
  if (!s.split && s.waves == 4) {
    // Two four-wave workgroups fit on a compute unit.  With more items
    // than such slots, exactly that many workgroups loop over the items,
    // fetching the next item's key tiles while they finish the current
    // one.  Below two items per slot each workgroup takes one or two, the
    // first dispatched first, in place of a second round of workgroups: 6,
    // 9 and 10 images at 384 px 29.4, 42.4 and 44.6 us against 30.7, 43.2
    // and 45.9; ViT-L/14 at 16 and 20 images 15.2 and 18.9 against 16.7
    // and 20.0.
    const int slots = 2 * compute_units;
    if (slots >= 16 && slots % 8 == 0 && s.items > slots) s.grid = slots;
  }
  return s;
}

}  // namespace vitattn

extern "C" const char* vitattn_strerror(int status) {
  switch (status) {
    case VITATTN_OK: return "success";
    case VITATTN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case VITATTN_ERR_BAD_SIZE: return "B, H or N is negative";
    case VITATTN_ERR_UNSUPPORTED_D: return "head dimension D must be 64 or 72";
    case VITATTN_ERR_BAD_SCALE: return "scale must be finite";
    case VITATTN_ERR_BAD_LAYOUT: return "unknown layout, or k/v passed with the packed layout";
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

extern "C" int vitattn_version(void) { return vitattn::kVersion; }
