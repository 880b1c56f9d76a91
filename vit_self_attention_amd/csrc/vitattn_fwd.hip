// Bidirectional multi-head self-attention forward for gfx950 (MI355X).
//
//   O = softmax(scale * Q K^T) V   per (image, head), softmax over keys.
//
// This is the fused attention core of a ViT / SigLIP vision encoder (the
// Pi0 Flash Attention tutorial, section 1: reordered computation, memory
// awareness and kernel fusion; section 3.2: fed from the fused qkv
// projection).  The kernel streams key/value tiles through LDS and keeps an
// online softmax in registers, so the N x N score matrix never reaches HBM.
//
// Work decomposition
//   * work items of (image, head, block of 32*NW queries); NW waves of 64
//     lanes, each wave owning 32 queries.  One workgroup per item; with
//     more items than four-wave workgroup slots, two four-wave workgroups
//     per compute unit loop over the items instead, fetching the next
//     item's tiles while they finish the current one;
//   * small grids split the keys instead (kSplit): the four waves share
//     one 32-query block, each reduces key tiles w, w+4, ... on its own
//     (more than one with kMulti, for more than 4 key tiles), and the
//     partial results merge through LDS;
//   * keys in tiles of 64, fetched cooperatively with 128-bit direct-to-LDS
//     loads into a ring of LDS stages (row-major K and V), three tiles ahead
//     of the tile being reduced, one barrier per tile;
//   * both products on 16-bit MFMA (bf16, or fp16 for fp16 inputs) with fp32
//     accumulation, in transposed form:
//       S^T = K Q^T       (v_mfma_f32_32x32x16_bf16; D = 72 adds a 32x32x8)
//       O^T += V^T P^T    (v_mfma_f32_32x32x16_bf16)
//     With S^T in the accumulator layout, lane l holds 16 keys of query
//     (l mod 32) per 32x32 block: the row max is mostly in-lane, and the
//     accumulator registers, converted to bf16, are directly the B operand
//     of the second product (keys permuted within each group of 16).  The
//     matching V^T operand comes from row-major V through the gfx950 LDS
//     transpose read (ds_read_b64_tr_b16), so V is never transposed in
//     memory;
//   * software pipeline inside each wave: the Q K^T products of tile j+1
//     are issued while the exponentials of tile j run on the VALU, and the
//     P V products of tile j overlap the row max of tile j+1;
//   * online softmax in base 2 with a lazy running max: the accumulator is
//     rescaled only when a row's max grows by more than 2^32 (fp16: 2^8);
//   * D = 72: the P V product runs three 32-row output tiles (d 0..95); the
//     spare row d = 72 reads a column of ones stored after each V row, so
//     the softmax denominator comes out of the same MFMA from the same bf16
//     weights that multiply V;
//   * tails: keys >= N of the last tile are fetched as copies of key N-1
//     (so row maxima are unchanged) and get zero weights; queries >= N run
//     on copies of query N-1 and are never stored, and a wave whose 32
//     queries all lie past N skips the products (it still fetches its share
//     of each tile and meets every barrier).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "vitattn.h"
#include "vitattn_internal.h"

namespace vitattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBlockN = 64;           // keys per tile
constexpr int kKStride = 72;          // K row stride in LDS (elements): 144 B
constexpr float kLog2e = 1.4426950408889634f;
// The running max is lazy: it moves (and the accumulator is rescaled) only
// when a row's max grows by more than 2^lazy.  Weights then stay below
// 2^lazy and row sums below N * 2^lazy, while rounding a weight to 16 bits is
// relative and so independent of the shift.  bf16 (fp32's exponent range):
// lazy = 32, so the fp32 sums of weight times value stay finite for any
// |V| below 2^128 / (N * 2^32), about 1e26 at N = 729 (measured: no cost
// against 2^64 at 384 px or N = 2048).  fp16 tops out near 2^16, so its
// weights are kept below 2^8 (and those under 2^-24 of the row max,
// negligible against it, flush to zero).
template <bool kF16>
constexpr float lazy_bound() { return kF16 ? 8.0f : 32.0f; }

// What the kernel works with; it arrives as scalar kernel arguments (see
// fwd_kernel) and the strides are derived from the layout in the kernel.
struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  // strides in elements; Q, K and V share theirs (both layouts)
  int64_t i_sb, i_sh;
  int64_t o_sb, o_sh;
  int i_st, o_st;  // token strides (a 64-token tile spans < 2 GiB)
  int H, N;
  int qblocks;     // query blocks per (image, head)
  int items;       // B * H * qblocks work items (image, head, query block)
  int grid;        // total workgroups: one per item, or fewer that loop over items
  float c;         // max(|scale|, tiny) * log2(e)
  uint32_t qsign;  // 0x80008000 when scale < 0: Q is negated instead
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest-even 16-bit values (bf16 or fp16), packed
// low/high into 32 bits (one v_cvt_pk_*_f32 on gfx950).
template <bool kF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (kF16) {
    f16x2 p;
    p[0] = static_cast<_Float16>(lo);
    p[1] = static_cast<_Float16>(hi);
    return __builtin_bit_cast(uint32_t, p);
  } else {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p;
    p[0] = static_cast<__bf16>(lo);
    p[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, p);
  }
}

// 16-bit input elements travel in bf16-typed vectors whatever their format;
// the MFMA wrappers reinterpret them for the fp16 instructions.
template <bool kF16>
__device__ __forceinline__ f32x16 mma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool kF16>
__device__ __forceinline__ f32x16 mma_32x32x8(bf16x4 a, bf16x4 b, f32x16 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
}
// acc + w.lo + w.hi for two packed 16-bit weights (v_dot2 with (1, 1))
template <bool kF16>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  if constexpr (kF16) {
    const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
  } else {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
  }
}

// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.  Fed two copies of v, the two results hold, in
// every lane, v of this lane and v of lane ^ 32 (in an order that depends on
// the half).  The elements are copied out as integers before the bit casts:
// a bit cast applied directly to a vector element reads element 0.
__device__ __forceinline__ void swap_halves(float v, float& x, float& y) {
  const uint32_t a = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  x = __builtin_bit_cast(float, r0);
  y = __builtin_bit_cast(float, r1);
}

// max(v[lane], v[lane ^ 32])
__device__ __forceinline__ float max_across_halves(float v) {
  float x, y;
  swap_halves(v, x, y);
  return fmaxf(x, y);
}

// v[lane] + v[lane ^ 32]
__device__ __forceinline__ float sum_across_halves(float v) {
  float x, y;
  swap_halves(v, x, y);
  return x + y;
}

// v of lane (lane mod 32): the lower half's value in both halves
__device__ __forceinline__ float lower_half_value(float v) {
  float x, y;
  swap_halves(v, x, y);
  return x;
}

// LDS transpose read: within each group of 16 lanes, lane 4a+b receives
// element b of the 8-byte rows that lanes 4j+a point at, for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// One direct-to-LDS fetch: every active lane copies 16 bytes from
// g + off (its own offset) into slot `lane` of the 64 x 16-byte LDS block at
// byte address lds_addr (wave-uniform, passed in M0).  Written as inline asm so that
// the compiler does not track it as an LDS store: its own tracking cannot
// tell the ring stage being filled from the stages being read and would put
// a full vector-memory wait before every LDS transpose read.  The kernel
// orders these fetches itself (vmcnt waits and a barrier before a stage is
// read; a stage is refilled only after the barrier that ends its reads; in
// the split kernel a wave reads only what it fetched, after its own vmcnt
// wait), and the memory clobber keeps LDS accesses from moving across it.
// Nothing else in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: the clobber is intended
__device__ __forceinline__ void dma16(const char* g, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  // one wait state between the M0 write and the instruction that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most n vector-memory instructions of this wave are in
// flight (vmcnt only: expcnt 7 and lgkmcnt 15 mean no wait on those).
// Loads, the direct-to-LDS fetches included, complete in issue order.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// n / d for 0 <= n < 2048 and 1 <= d < 2048, as floor(n * rcp(d) + 2^-12)
// with the hardware reciprocal (v_rcp_f32, within an ulp): a handful of VALU
// operations in place of the thirty-odd dependent instructions of a general
// 32-bit division, which sit at the start of every workgroup.  Over that
// range the bias exceeds the product's error, so an exact quotient is not
// rounded down, and bias plus error stay below 1/d, the least distance from
// a non-integer n/d up to the next integer: the floor is exact (checked for
// every such n and d, with reciprocals up to two ulp from 1/d, by the host
// tests).
__device__ __forceinline__ int div_small(int n, int d) {
  return static_cast<int>(
      __builtin_fmaf(static_cast<float>(n), __builtin_amdgcn_rcpf(static_cast<float>(d)), 0x1p-12f));
}

// Workgroup id -> logical tile id.  Workgroups are dispatched round-robin
// over the 8 XCDs (id mod 8); this bijection gives each XCD a contiguous
// range of logical tiles, so the query blocks of one (image, head) -- which
// read the same K and V -- share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  const int q = grid >> 3, r = grid & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + (x < r ? x : r) + i;
}

// kSplit (NW = 4): the waves of a workgroup share one block of 32 queries,
// wave w fetches and reduces key tile w on its own (and, with kMulti, tiles
// w + 4, w + 8, ... after it, in the same LDS stage), and the partial
// results are merged through LDS at the end.  This gives four times the
// waves for grids too small to fill the chip.
template <int D, int NW, bool kSplit, bool kF16, bool kMulti = false>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(int grid, int qblocks, int H, int N_, int i_st,
                                                      float cs, const uint16_t* q, const uint16_t* k,
                                                      const uint16_t* v, uint16_t* o, int items) {
  // The arguments are scalars, all but `items` (14 dwords) preloaded into
  // SGPRs at wave launch instead of read from the argument buffer; the
  // looping kernel alone reads `items`.  cs is the softmax factor c, negated
  // when the scale is negative (Q is then negated instead).  The strides
  // follow from the layout: separate [B,H,N,D] rows are D apart, packed
  // [B,N,3,H,D] rows 3*H*D, and the output is [B,H,N,D] or [B,N,H,D].
  // The split kernel's qblocks and H carry, above their low 8 and 11 bits,
  // the multipliers ceil(2^16 / qblocks) and ceil(2^20 / H) that divide by
  // them (see launch).
  const int qblocks_ = kSplit ? (qblocks & 0xff) : qblocks;
  const int H_ = kSplit ? (H & 0x7ff) : H;
  KernelArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.i_st = i_st;
  a.H = H_;
  a.N = N_;
  a.qblocks = qblocks_;
  a.items = items;
  a.grid = grid;
  a.c = __builtin_fabsf(cs);
  a.qsign = cs < 0.f ? 0x80008000u : 0u;
  {
    const bool sep = i_st == D;
    const int64_t nd = static_cast<int64_t>(N_) * D;
    a.i_sh = sep ? nd : D;
    a.i_sb = sep ? H_ * nd : static_cast<int64_t>(N_) * i_st;
    a.o_sb = H_ * nd;
    a.o_sh = sep ? nd : D;
    a.o_st = sep ? D : H_ * D;
  }
  constexpr bool kOnesRow = (D % 32) != 0;          // D = 72
  constexpr int kOutTiles = kOnesRow ? 3 : 2;
  // V row: D values (+ [1,0,..,0] for D = 72) in a 160-byte row; with the key
  // order below this stride makes the transpose reads free of bank conflicts
  constexpr int kVStride = 80;
  constexpr int kKTile = kBlockN * kKStride;        // elements
  constexpr int kVTile = kBlockN * kVStride;
  constexpr int kStageElems = kKTile + kVTile;
  // LDS ring: tile t lives in stage t % kStages and is fetched kStages-1
  // tiles ahead of the one being reduced; two workgroups share a compute unit.
  constexpr int kStages = 4;
  // stage of stream tile s >= 0 (unsigned, so the modulo is a mask)
  auto stage_of = [](int s) { return static_cast<int>(static_cast<unsigned>(s) % kStages); };
  static_assert(NW <= 4, "the LDS ring is sized for two workgroups of at most four waves");
  // Direct-to-LDS fetches: each wave instruction moves 64 lanes x 16 B into
  // 64 consecutive 16-byte LDS slots, 9 per K row and 10 per V row.  Slots
  // past the D values of a row receive a copy of the row's last chunk: they
  // are never read, except V's slot 9 for D = 72, which is rewritten with
  // [1, 0, ..., 0] once the tile has landed (write_ones below).
  constexpr int kKSlotsRow = kKStride / 8, kVSlotsRow = kVStride / 8;
  constexpr int kKInstr = kBlockN * kKSlotsRow / 64;
  constexpr int kVInstr = kBlockN * kVSlotsRow / 64;
  constexpr int kInstr = kKInstr + kVInstr;
  constexpr int kPerWave = (kInstr + NW - 1) / NW;   // fetch instructions of the busiest wave
  constexpr int kMinPerWave = kInstr / NW;           // ... and of the least busy one
  static_assert(kBlockN * kKSlotsRow % 64 == 0 && kBlockN * kVSlotsRow % 64 == 0, "slots");

  // the ring, then a 1 KB sink for the filler fetches of waves with fewer
  // fetch instructions in a steady step (never read)
  constexpr int kSinkElems = 512;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStages * kStageElems + kSinkElems];
  // byte address of lds in the LDS aperture (what M0 takes)
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)lds));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
  const int col = lane & 31;   // query within the wave (MFMA column)
  const int half = lane >> 5;  // which half of the MFMA K dimension this lane feeds

  const int N = a.N;
  const int ntiles = (N + kBlockN - 1) / kBlockN;

  // ---- work items.  With one workgroup per item, item = xcd_remap(block).
  // With fewer workgroups (two per compute unit, a whole number per XCD),
  // each loops over items in rounds: XCD x owns a contiguous range of items
  // and round r gives its workgroup l the item lo + r*G + l, so the query
  // blocks of one (image, head), which read the same K and V, run at about
  // the same time in that XCD's L2.  Of the two workgroups on a compute
  // unit, the one dispatched first (block < grid/2) wins most issue
  // conflicts and runs about 1.2 times faster: the last rounds, past
  // 0.9 times the average number of items, go to those workgroups only.
  // With fewer than two items per workgroup the second round is spread over
  // all of them instead, the first dispatched first, so none takes three.
  int it0 = 0, lo = 0, gx = 1, ky = 1, lx = 0;
  bool single = true;
  int nitems = 1;
  if (kSplit || a.grid >= a.items) {  // the split kernel never loops
    it0 = xcd_remap(blockIdx.x, a.grid);
  } else {
    single = false;
    const int x = blockIdx.x & 7;
    lx = blockIdx.x >> 3;
    gx = a.grid >> 3;
    const int per = a.items >> 3, rem = a.items & 7;
    lo = x * per + (x < rem ? x : rem);
    const int nx = per + (x < rem ? 1 : 0);
    ky = (9 * nx + 5 * gx) / (10 * gx);  // 0.9 * nx / gx, rounded, at most nx / gx
    if (ky > nx / gx) ky = nx / gx;
    it0 = lo + lx;
    nitems = ky;
    if (nx < 2 * gx) {
      nitems = 1 + (lx < nx - gx ? 1 : 0);  // ky = 1: item_at(1) = lo + gx + lx
    } else if (lx < gx / 2) {
      const int left = nx - ky * gx - lx;
      nitems += left > 0 ? (left + gx / 2 - 1) / (gx / 2) : 0;
    }
  }
  // item of round r
  auto item_at = [&](int r) {
    if (single) return it0;
    return r < ky ? lo + r * gx + lx : lo + ky * gx + (r - ky) * (gx / 2) + lx;
  };
  // (image, head, query block) of an item
  auto coords = [&](int item, int& bi, int& hi_, int& qbi) {
    const int bh = item / a.qblocks;
    qbi = item - bh * a.qblocks;
    bi = bh / a.H;
    hi_ = bh - bi * a.H;
  };
  int b, h, qb;
  // the first item's, on the path to the first fetch
  if constexpr (kSplit) {
    // q = (n * ceil(2^k / d)) >> k is n / d whenever n * d < 2^k: here
    // every item * qblocks < 2^16 and (image, head) * H < 2^20, and the
    // 32-bit products do not overflow (launch checks both)
    const int bh = static_cast<int>((static_cast<uint32_t>(it0) * (static_cast<uint32_t>(qblocks) >> 8)) >> 16);
    b = static_cast<int>((static_cast<uint32_t>(bh) * (static_cast<uint32_t>(H) >> 11)) >> 20);
    qb = it0 - bh * a.qblocks;
    h = bh - b * a.H;
  } else if (a.items < 2048) {
    // below 2048 items every quotient is a small one; the two quotients
    // (qblocks * H <= items) are independent, so their latencies overlap
    const int bh = div_small(it0, a.qblocks);
    b = div_small(it0, a.qblocks * a.H);
    qb = it0 - bh * a.qblocks;
    h = bh - b * a.H;
  } else {
    coords(it0, b, h, qb);
  }
  const uint16_t* kbase = a.k + b * a.i_sb + h * a.i_sh;
  const uint16_t* vbase = a.v + b * a.i_sb + h * a.i_sh;

  // ---- constant tail of each V row (D = 72): d = 72 holds 1, d = 73..79
  // hold 0.  Every wave writes the whole column of a stage itself (lane =
  // row) after the stage's tile has landed and before it reads the tile's
  // V, so no other wave's write needs to be visible to it.
  auto write_ones = [&](int stage) __attribute__((always_inline)) {
    if constexpr (kOnesRow) {
      const u32x4 w = {kF16 ? 0x3c00u : 0x3f80u, 0u, 0u, 0u};  // 1.0
      *reinterpret_cast<u32x4*>(&lds[stage * kStageElems + kKTile + lane * kVStride + 72]) = w;
    }
  };

  // ---- this lane's query row as the B operand of S^T = K Q^T
  auto first_query = [&](int qb_) { return kSplit ? qb_ * 32 : qb_ * (32 * NW) + wave * 32; };
  // loads the query row of this lane for item (b_, h_, qb_) into dq, dqt as
  // stored (rows past N load row N-1: their columns of S are never stored
  // and touch no other column); sign_q then applies the sign of the scale
  auto load_q = [&](int b_, int h_, int qb_, bf16x8* dq, bf16x4& dqt) __attribute__((always_inline)) {
    const int q_ = first_query(qb_) + col;
    const int qi_ = q_ < N ? q_ : N - 1;
    const uint16_t* qrow = a.q + b_ * a.i_sb + h_ * a.i_sh + static_cast<int64_t>(qi_) * a.i_st;
#pragma unroll
    for (int s = 0; s < 4; ++s) dq[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * half);
    if constexpr (D == 72) dqt = *reinterpret_cast<const bf16x4*>(qrow + 64 + 4 * half);
  };
  auto sign_q = [&](bf16x8* dq, bf16x4& dqt) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) dq[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, dq[s]) ^ a.qsign);
    if constexpr (D == 72) dqt = __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, dqt) ^ a.qsign);
  };
  int q0 = first_query(qb);
  int qi = q0 + col;
  bool wave_active = q0 < N;
  bf16x8 qf[4];
  bf16x4 qt = {};
  if constexpr (!kSplit) {  // the split kernel stages its query rows through LDS
    load_q(b, h, qb, qf, qt);
    sign_q(qf, qt);
  }
  int nb = b, nh = h, nqb = qb;  // next item (the current one after the last)

  // ---- direct-to-LDS tile fetch.  Fetch instruction i of this wave is
  // number I = i*NW + wave of the tile: I < kKInstr fills K slots, the rest
  // V slots.  Slot s of a row-major LDS tile holds row s / slots_per_row,
  // 16-byte column s % slots_per_row (clamped to the last chunk of D).  In
  // the last tile, rows past N repeat row N-1 (finite data that a zero
  // weight removes).
  const int st32 = a.i_st;
  // row and clamped 16-byte column of this lane's slot in fetch instruction I
  auto slot_rc = [&](int I, int& row, int& cc) __attribute__((always_inline)) {
    const bool is_k = I < kKInstr;
    const int slot = (is_k ? I : I - kKInstr) * 64 + lane;
    const int per_row = is_k ? kKSlotsRow : kVSlotsRow;
    row = slot / per_row;
    const int c0 = slot - row * per_row;
    cc = c0 < D / 8 ? c0 : D / 8 - 1;
  };
  uint32_t f_off[kPerWave];  // byte offset of this lane's chunk from the tile's first row
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int I = i * NW + wave;
    int row, cc;
    slot_rc(I, row, cc);
    f_off[i] = static_cast<uint32_t>((row * st32 + cc * 8) * 2);
  }
  // issues this wave's fetch instructions for key tile t of the (image,
  // head) whose K and V start at kb_ptr and vb_ptr, into LDS stage `st`, as
  // straight-line code (every lane of every instruction fetches; the tail
  // is one uniform branch)
  auto fetch_tile_at = [&](const uint16_t* kb_ptr, const uint16_t* vb_ptr, int t, int st)
                           __attribute__((always_inline)) {
    const int kb = t * kBlockN;
    const char* gk = reinterpret_cast<const char*>(kb_ptr + static_cast<int64_t>(kb) * a.i_st);
    const char* gv = reinterpret_cast<const char*>(vb_ptr + static_cast<int64_t>(kb) * a.i_st);
    const uint32_t stage = lds_base + 2 * st * kStageElems;
    auto slot_addr = [&](int I) {
      return stage + 2 * (I < kKInstr ? I * 512 : kKTile + (I - kKInstr) * 512);
    };
    if (kb + kBlockN <= N) {
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int I = i * NW + wave;
        if (i >= kMinPerWave && I >= kInstr) continue;  // only the last round can be short
        dma16(I < kKInstr ? gk : gv, f_off[i], slot_addr(I));
      }
    } else {
      const int last = N - 1 - kb;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int I = i * NW + wave;
        if (i >= kMinPerWave && I >= kInstr) continue;
        const bool is_k = I < kKInstr;
        int row, cc;
        slot_rc(I, row, cc);
        const int r = row < last ? row : last;
        dma16(is_k ? gk : gv, static_cast<uint32_t>((r * st32 + cc * 8) * 2), slot_addr(I));
      }
    }
  };
  // ---- the tile stream.  The workgroup reduces the key tiles of its items
  // one after another; stream tile s (tile s % ntiles of the workgroup's
  // item s / ntiles) lives in LDS stage s % kStages and is fetched
  // kStages-1 tiles ahead, across item boundaries.
  const int stream_len = nitems * ntiles;
  int f_s = 0, f_t = 0, f_r = 0;  // next stream tile to fetch: tile f_t of round f_r
  const uint16_t* f_kb = kbase;
  const uint16_t* f_vb = vbase;
  auto fetch_next = [&]() __attribute__((always_inline)) {
    if (f_s >= stream_len) return;
    fetch_tile_at(f_kb, f_vb, f_t, stage_of(f_s));
    ++f_s;
    if (++f_t == ntiles && f_s < stream_len) {
      f_t = 0;
      ++f_r;
      int bn, hn, qn;
      coords(item_at(f_r), bn, hn, qn);
      f_kb = a.k + bn * a.i_sb + hn * a.i_sh;
      f_vb = a.v + bn * a.i_sb + hn * a.i_sh;
    }
  };
  // The fetch of a steady step (see step): a tile of the item being fetched
  // other than its last (so a full one), so none of fetch_next's checks (end
  // of stream, tail rows, switch to the next item) can be taken.  The step
  // issues this wave's instructions one at a time between its first matrix
  // products (fetch_steady_one(i), i < kPerWave), then advances the stream
  // (fetch_steady_done).  Issued together right after the barrier, the
  // tile's 19 instructions queue at the compute unit's texture addresser
  // and hold every wave for about a fifth of the step.  Waves without an
  // i-th instruction repeat their first one into the sink, so every wave
  // issues kPerWave of them with no branch (a branch in the chunk sequence
  // lets the compiler sink the exponentials out of it).
  auto fetch_steady_one = [&](int i) __attribute__((always_inline)) {
    const char* gk = reinterpret_cast<const char*>(f_kb + static_cast<int64_t>(f_t * kBlockN) * a.i_st);
    const char* gv = reinterpret_cast<const char*>(f_vb + static_cast<int64_t>(f_t * kBlockN) * a.i_st);
    const uint32_t stage = lds_base + 2 * stage_of(f_s) * kStageElems;
    const int I = i * NW + wave;
    if (i < kMinPerWave) {
      dma16(I < kKInstr ? gk : gv, f_off[i], stage + 2 * (I < kKInstr ? I * 512 : kKTile + (I - kKInstr) * 512));
    } else {
      const bool real = I < kInstr;
      const uint32_t sink = lds_base + 2 * kStages * kStageElems;
      const char* src = real ? (I < kKInstr ? gk : gv) : (wave < kKInstr ? gk : gv);
      dma16(src, real ? f_off[i] : f_off[0],
            real ? stage + 2 * (I < kKInstr ? I * 512 : kKTile + (I - kKInstr) * 512) : sink);
    }
  };
  auto fetch_steady_done = [&]() __attribute__((always_inline)) {
    ++f_s;
    ++f_t;
  };
  // Waits until the fetches of all but the last `tiles_in_flight` (0 or 1)
  // tiles issued by this wave have landed (vector-memory counter only; a
  // wave issues at least kMinPerWave fetches per tile, and no other load
  // after them), then meets the rest of the workgroup.  The memory clobber
  // keeps LDS accesses after it.
  auto wait_fetch_and_sync = [&](int tiles_in_flight) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    if (tiles_in_flight == 0) {
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<kMinPerWave>();
    }
    asm volatile("s_barrier" ::: "memory");
  };
  // tiles fetched after tile t (0 or 1 with a four-stage ring), at the point
  // where the fetch of tile `issued` is the last one
  auto after = [&](int t, int issued) { return issued > t ? issued - t : 0; };

  // ---- key order.  Row i of each 32-key block of S^T holds key
  // krow(i) = 16*(i/16) + perm16(i%16), perm16(8m + 4h + j) = 8m + 2j + h:
  // a transpose read then touches keys {0,2,4,6} (+8m) in one half of the
  // wave and {1,3,5,7} in the other, whose 64-byte V row segments land in
  // disjoint LDS banks at a 160-byte row stride.  The order is invisible
  // outside: K rows and V rows are read in the same order.
  auto krow = [](int i) { return 16 * (i >> 4) + 8 * ((i >> 3) & 1) + 2 * (i & 3) + ((i >> 2) & 1); };
  // ---- per-lane LDS read offsets (elements)
  // K operand (A of S^T = K Q^T): key row 32*blk + krow(col), columns 16*st + 8*half
  const int k_off = krow(col) * kKStride + 8 * half;
  const int k_off_tail = krow(col) * kKStride + 64 + 4 * half;
  // V^T operand (A of O^T = V^T P^T) via transpose reads: this lane names
  // key row 16t + krow(4*half + ((lane>>2)&3)) (+8 for the second read) and
  // column 32*mt + 16*((lane>>4)&1) + 4*(lane&3).  The row-sum tile (mt = 2,
  // D = 72) has 9 used rows (d = 64..72): the 16-lane groups of rows 64..79
  // read columns 64 + 4*(lane&3), those of rows 80..95 (never stored) the
  // zero columns 76..79, which lowers the matrix cores' power draw and with
  // it the clock penalty (about 1% at 384 px, the same output bits).
  const int v_row = krow(4 * half + ((lane >> 2) & 3));
  const int v_off = v_row * kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int v_off_tail = v_row * kVStride + (((lane >> 4) & 1) ? 76 : 64 + 4 * (lane & 3));

  const float c = a.c;

  // ---- building blocks of one key tile
  // K operand of Q K^T step i (i < 8: columns 16*(i/2) of key block i%2;
  // D = 72 adds steps 8, 9 over columns 64..71 with the 32x32x8 shape)
  auto k_read = [&](const uint16_t* kt, int i) {
    return *reinterpret_cast<const bf16x8*>(kt + k_off + 32 * (i & 1) * kKStride + 16 * (i >> 1));
  };
  auto k_read_tail = [&](const uint16_t* kt, int blk) {
    return *reinterpret_cast<const bf16x4*>(kt + k_off_tail + 32 * blk * kKStride);
  };
  auto qk_plain = [&](const uint16_t* kt, f32x16* s) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[blk][r] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s[i & 1] = mma_32x32x16<kF16>(k_read(kt, i), qf[i >> 1], s[i & 1]);
    if constexpr (D == 72) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        s[blk] = mma_32x32x8<kF16>(k_read_tail(kt, blk), qt, s[blk]);
    }
  };
  // S^T of one 32-key block (rows 32*blk .. 32*blk+31 of the tile)
  auto qk_block = [&](const uint16_t* kt, f32x16* s, int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[blk][r] = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) s[blk] = mma_32x32x16<kF16>(k_read(kt, 2 * st + blk), qf[st], s[blk]);
    if constexpr (D == 72) s[blk] = mma_32x32x8<kF16>(k_read_tail(kt, blk), qt, s[blk]);
  };
  // V^T operand of P V step idx = t*kOutTiles + mt (keys 16t.., output rows 32mt..)
  auto v_read = [&](const uint16_t* vt, int idx) {
    const int t = idx / kOutTiles, mt = idx % kOutTiles;
    const int off = (kOnesRow && mt == 2) ? v_off_tail : v_off + 32 * mt;
    const uint16_t* p = vt + off + 16 * t * kVStride;
    const u32x2 lo = lds_read_tr(p);
    const u32x2 hi = lds_read_tr(p + 8 * kVStride);
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, w);
  };
  // s[blk][r] is the logit of key kb + 32*blk + krow(8*(r/4) + 4*half + (r%4));
  // element e = 16*blk + r, and P V step t uses elements 8t .. 8t+7.
  auto key_of = [&](int e) { return 32 * (e >> 4) + krow(8 * ((e & 15) >> 2) + 4 * half + (e & 3)); };
  // partial row max over elements 4g .. 4g+3
  auto max4 = [&](const f32x16* s, int g) {
    const f32x16& v = s[g >> 2];
    const int r = 4 * (g & 3);
    return fmaxf(fmaxf(v[r], v[r + 1]), fmaxf(v[r + 2], v[r + 3]));
  };
  auto rowmax = [&](const f32x16* s) {
    float m[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) m[g] = max4(s, g);
    return max_across_halves(
        fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7]))));
  };
  constexpr float kLazy = lazy_bound<kF16>();
  float psum = 0.f;  // D = 64: row sum of the bf16 weights (dot products with ones)
  f32x16 acc[kOutTiles];
#pragma unroll
  for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float mx = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;  // per-lane partial row sum (D = 64)

  // (split kernel with kMulti: the K rows of the wave's next tile are in
  // flight behind this tile's V rows)
  bool pend_k = false;
  // ---- one key tile j.  `cur` holds the logits of tile j; when kNext,
  // the logits of tile j+1 go to `nxt` and their row max to mx.  kRagged
  // (last tile, N not a multiple of 64) zeroes the weights of keys >= N.
  // The body is issued in chunks fenced by sched_barrier: each chunk pairs
  // one MFMA with the LDS reads of the MFMA two steps later and a share of
  // the VALU work (exponentials, bf16 packing, maxima), so the VALU runs
  // while the matrix core works.
  // j is the tile's index in its item, gs its index in the tile stream
  // (gs = j for the split kernel, whose stage of tile j is stage j).
  // kSteady: a step in the middle of an item whose fetch is a tile of the
  // same item other than its last (j + 4 < ntiles): the fetch, the write of
  // the next stage's ones column and the wait at the end are then
  // unconditional, with no branch and little scalar work.
  auto step = [&](int j, int gs, f32x16* cur, f32x16* nxt, auto kNextC, auto kRaggedC,
                  auto kHalfC, auto kSteadyC) __attribute__((always_inline)) {
    constexpr bool kSteady = decltype(kSteadyC)::value;
    constexpr bool kNext = decltype(kNextC)::value;
    static_assert(!kSteady || kNext, "steady steps have a next tile");
    constexpr bool kRagged = decltype(kRaggedC)::value;
    // kHalf (the item's last step only): the tile holds at most 32 keys, so
    // only its first 32-key block is weighted and multiplied into P V; its
    // keys 32..63 would all get zero weight.  (Q K^T of the tile ran a step
    // earlier over both blocks.)
    constexpr bool kThisHalf = decltype(kHalfC)::value;
    static_assert(!(kThisHalf && kNext), "only the last step reduces a half tile");
    if constexpr (kSteady) {
      write_ones(stage_of(gs + 1));
    } else if constexpr (!kSplit) {
      // stage (gs-1) % kStages held stream tile gs-1, whose reads all ended
      // before the last barrier; it is refilled with stream tile gs + kStages - 1
      fetch_next();
      // stream tile gs+1 landed before the last barrier; its V is read next step
      if (gs + 1 < stream_len) write_ones(stage_of(gs + 1));
    }

    if (wave_active) {
      // lazy running max: move it (and rescale) only when some row's max
      // grew by more than 2^kLazy
      const float m_cand = mx * c;
      const bool grow = m_cand > m_run + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = grow ? fast_exp2(m_run - m_cand) : 1.f;
        m_run = grow ? m_cand : m_run;
#pragma unroll
        for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
        l_run *= alpha;
      }
      const float neg_m = -m_run;
      const int kb = j * kBlockN;
      const uint16_t* kt = lds + stage_of(gs + 1) * kStageElems;
      const uint16_t* vt = lds + stage_of(gs) * kStageElems + kKTile;

      float p[32];
      uint32_t w[16];
      auto do_exp = [&](int e) {
        p[e] = fast_exp2(__builtin_fmaf(cur[e >> 4][e & 15], c, neg_m));
        if constexpr (kRagged) p[e] = kb + key_of(e) < N ? p[e] : 0.f;
        if (e & 1) {
          const int k = e >> 1;
          w[k] = pack2<kF16>(p[2 * k], p[2 * k + 1]);
          if constexpr (!kOnesRow)
            psum = add_pair<kF16>(w[k], psum);
        }
      };
      auto pb = [&](int t) {
        const u32x4 v = {w[4 * t], w[4 * t + 1], w[4 * t + 2], w[4 * t + 3]};
        return __builtin_bit_cast(bf16x8, v);
      };

      // phase 1: Q K^T of tile j+1 with the weights of keys 0..47 of tile j
      constexpr int kQk = D == 72 ? 10 : 8;
      if constexpr (kNext) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) nxt[blk][r] = 0.f;
        bf16x8 ko[8];
        bf16x4 ko4[2];
        auto fetch_k = [&](int i) {
          if (i < 8) ko[i] = k_read(kt, i);
          else ko4[i - 8] = k_read_tail(kt, i - 8);
        };
        fetch_k(0);
        fetch_k(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kQk; ++i) {
          if (i + 2 < kQk) fetch_k(i + 2);
          if (i < 8)
            nxt[i & 1] = mma_32x32x16<kF16>(ko[i], qf[i >> 1], nxt[i & 1]);
          else
            nxt[i & 1] = mma_32x32x8<kF16>(ko4[i - 8], qt, nxt[i & 1]);
#pragma unroll
          for (int e = 24 * i / kQk; e < 24 * (i + 1) / kQk; ++e) do_exp(e);
          // a steady step's fetch, spread evenly over the chunks
          if constexpr (kSteady) {
#pragma unroll
            for (int f = 0; f < kPerWave; ++f)
              if (f * kQk / kPerWave == i) fetch_steady_one(f);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < (kThisHalf ? 16 : 24); ++e) do_exp(e);
      }

      // phases 2 and 3: P V of tile j; the remaining weights ride along the
      // first half, the row max of tile j+1 the second half
      // (a half tile: keys 0..31 only, all weighted in phase 1)
      constexpr int kPv = (kThisHalf ? 2 : 4) * kOutTiles, kHalfPv = 2 * kOutTiles;
      bf16x8 vo[kPv];
      vo[0] = v_read(vt, 0);
      vo[1] = v_read(vt, 1);
      float gmax = -__builtin_inff();  // running max of the logits of tile j+1
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kPv; ++i) {
        if constexpr (kSplit && !kThisHalf) {
          // the split kernel enters with V rows 0..31 landed; rows 32..63
          // (keys of steps t = 2, 3) are waited for before their first read
          if (i + 2 == kHalfPv) {
            if constexpr (kMulti) {
              if (pend_k) wait_vmcnt<kKInstr>();
              else wait_vmcnt<0>();
            } else {
              wait_vmcnt<0>();
            }
            asm volatile("" ::: "memory");
            if (half == 1) write_ones(stage_of(gs));
          }
        }
        if (i + 2 < kPv) vo[i + 2] = v_read(vt, i + 2);
        const int t = i / kOutTiles, mt = i % kOutTiles;
        acc[mt] = mma_32x32x16<kF16>(vo[i], pb(t), acc[mt]);
        if (i < kHalfPv) {
          if constexpr (!kThisHalf) {
#pragma unroll
            for (int e = 24 + 8 * i / kHalfPv; e < 24 + 8 * (i + 1) / kHalfPv; ++e) do_exp(e);
          }
        } else if constexpr (kNext) {
          const int ii = i - kHalfPv;
#pragma unroll
          for (int g = 8 * ii / kHalfPv; g < 8 * (ii + 1) / kHalfPv; ++g) {
            // two three-input maxima per group of four logits
            const f32x16& v = nxt[g >> 2];
            const int r = 4 * (g & 3);
            gmax = fmaxf(fmaxf(gmax, v[r]), v[r + 1]);
            gmax = fmaxf(fmaxf(gmax, v[r + 2]), v[r + 3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kNext) {
        mx = max_across_halves(gmax);
      }
      if constexpr (!kOnesRow) {
        l_run += psum;
        psum = 0.f;
      }
    }

    if constexpr (kSteady) {
      if (!wave_active) {  // (a wave with no queries skipped the chunks above)
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) fetch_steady_one(i);
      }
      fetch_steady_done();
    }
    if constexpr (!kSplit && !kNext) {
      // the item's last tile is reduced: start loading the next item's query
      // rows into qf, qt (after the last item this reloads that item's rows,
      // which are not used again)
      load_q(nb, nh, nqb, qf, qt);
    }
    // stream tile gs+2 must have landed before the next step reads its K,
    // and every wave must be done with stage gs % kStages before it is refilled
    if constexpr (kSteady) {
      // tile gs+3 (fetched this step, kPerWave instructions from every
      // wave) stays in flight
      asm volatile("" ::: "memory");
      wait_vmcnt<kPerWave>();
      asm volatile("s_barrier" ::: "memory");
    } else if constexpr (!kSplit) {
      if constexpr (kNext) {
        if (gs + 1 < stream_len) wait_fetch_and_sync(after(gs + 2, f_s - 1));
      } else {
        // Everything this wave has in flight, the next item's query rows
        // included, lands here (its last fetch was issued a step ago): the
        // compiler's own waits for those rows then find nothing left to wait
        // for in the next item, where a count of its loads alone would also
        // wait for fetches issued after them.
        wait_fetch_and_sync(0);
      }
    }
  };

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  const bool ragged = N % kBlockN != 0;
  // the last key tile holds at most 32 keys
  const bool half_tail = ragged && N % kBlockN <= 32;
  f32x16 sa[2], sb[2];

  if constexpr (kSplit) {
    // ---- wave w alone fetches key tile w into stage w and reduces it; no
    // other wave touches that stage, so nothing is shared before the merge.
    // The wave fetches the block's 32 query rows (row r at kKStride
    // elements; rows past N repeat row N-1) into the stage's V region with
    // its K rows, takes the query rows into registers once they land, and
    // only then fetches its V rows over them: Q K^T runs while V is in
    // flight.
    const int my = wave;
    if (wave_active && my < ntiles) {
      const uint32_t stage = lds_base + 2 * my * kStageElems;
      // fetch instructions [lo, hi) of tile t (I < kKInstr fill K slots)
      auto fetch_own = [&](int t, int lo, int hi) __attribute__((always_inline)) {
        const int kb0 = t * kBlockN;
        const char* gk = reinterpret_cast<const char*>(kbase + static_cast<int64_t>(kb0) * a.i_st);
        const char* gv = reinterpret_cast<const char*>(vbase + static_cast<int64_t>(kb0) * a.i_st);
        const int last = N - 1 - kb0;
#pragma unroll
        for (int I = lo; I < hi; ++I) {
          int row, cc;
          slot_rc(I, row, cc);
          const int r = row < last ? row : last;
          dma16(I < kKInstr ? gk : gv, static_cast<uint32_t>((r * st32 + cc * 8) * 2),
                stage + 2 * (I < kKInstr ? I * 512 : kKTile + (I - kKInstr) * 512));
        }
      };
      constexpr int kQInstr = (32 * kKSlotsRow + 63) / 64;
      static_assert(kQInstr * 512 <= kVTile, "the query rows fit in a V tile");
      {
        const char* gq = reinterpret_cast<const char*>(a.q + b * a.i_sb + h * a.i_sh +
                                                       static_cast<int64_t>(q0) * a.i_st);
#pragma unroll
        for (int i = 0; i < kQInstr; ++i) {
          const int slot = i * 64 + lane;
          int row = slot / kKSlotsRow;
          const int c0 = slot - row * kKSlotsRow;
          const int cc = c0 < D / 8 ? c0 : D / 8 - 1;
          row = row < 32 ? row : 31;  // slots past the block: a copy, never read
          row = q0 + row < N ? row : N - 1 - q0;
          dma16(gq, static_cast<uint32_t>((row * st32 + cc * 8) * 2), stage + 2 * (kKTile + i * 512));
        }
      }
      fetch_own(my, 0, kKInstr);
      wait_vmcnt<kKInstr>();  // the query rows landed
      asm volatile("" ::: "memory");
      {
        const uint16_t* qr = lds + my * kStageElems + kKTile + col * kKStride;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s + 8 * half);
        if constexpr (D == 72) qt = *reinterpret_cast<const bf16x4*>(qr + 64 + 4 * half);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the V rows land on them
      sign_q(qf, qt);
      fetch_own(my, kKInstr, kInstr);
      // K rows 0..35 (the first five fetches) carry key block 0, the rest
      // block 1; V rows 0..31 (the first five) keys 0..31 of P V
      constexpr int kHalfFetch = 5;
      static_assert(kHalfFetch * 64 >= 32 * kKSlotsRow && kHalfFetch * 64 == 32 * kVSlotsRow,
                    "five fetches cover 32 rows of K and exactly 32 of V");
      wait_vmcnt<kVInstr + kKInstr - kHalfFetch>();
      asm volatile("" ::: "memory");
      qk_block(lds + my * kStageElems, sa, 0);
      wait_vmcnt<kVInstr>();  // the K rows landed
      asm volatile("" ::: "memory");
      qk_block(lds + my * kStageElems, sa, 1);
      mx = rowmax(sa);
      asm volatile("" ::"v"(mx));  // the row max is taken before the wait below
      // (kMulti) the next tile's K rows go out now, into the K region this
      // tile's Q K^T has finished reading, and land during its P V
      auto fetch_next_k = [&](int t) __attribute__((always_inline)) {
        if constexpr (kMulti) {
          pend_k = t + 4 < ntiles;
          if (pend_k) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            fetch_own(t + 4, 0, kKInstr);
          }
        }
      };
      auto wait_v_half = [&]() __attribute__((always_inline)) {
        if (pend_k) wait_vmcnt<kVInstr - kHalfFetch + kKInstr>();
        else wait_vmcnt<kVInstr - kHalfFetch>();  // V rows 0..31 landed
        asm volatile("" ::: "memory");
      };
      fetch_next_k(my);
      wait_v_half();
      if (half == 0) write_ones(my);  // rows 0..31 (lane = row); rows 32..63 in the step
      if (ragged && my == ntiles - 1) step(my, my, sa, sb, False{}, True{}, False{}, False{});
      else step(my, my, sa, sb, False{}, False{}, False{}, False{});
      if constexpr (kMulti) {
        // the wave's further tiles my + 4, my + 8, ... in the same stage
        // (tile t lives in stage t % 4 = wave), one after another: K, then
        // V, with Q K^T of each 32-key block as soon as its K rows land
        // the V rows of tile my + 4 follow its K rows, after this tile's P V
        if (pend_k) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the last tile's reads returned
          fetch_own(my + 4, kKInstr, kInstr);
        }
        for (int t = my + 4; t < ntiles; t += 4) {
          wait_vmcnt<kVInstr + kKInstr - kHalfFetch>();
          asm volatile("" ::: "memory");
          qk_block(lds + my * kStageElems, sa, 0);
          wait_vmcnt<kVInstr>();
          asm volatile("" ::: "memory");
          qk_block(lds + my * kStageElems, sa, 1);
          mx = rowmax(sa);
          asm volatile("" ::"v"(mx));
          fetch_next_k(t);
          wait_v_half();
          if (half == 0) write_ones(my);
          if (ragged && t == ntiles - 1) step(t, t, sa, sb, False{}, True{}, False{}, False{});
          else step(t, t, sa, sb, False{}, False{}, False{}, False{});
          if (pend_k) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            fetch_own(t + 4, kKInstr, kInstr);
          }
        }
      }
    }
    // ---- merge the partial results of the waves (each: running max m,
    // accumulator, and for D = 64 the partial row sum) through LDS.  Wave w
    // writes its part into its own stage, which no other wave has touched,
    // laid out [group of 4 registers][lane][4] so every access is 1 KB
    // contiguous; one barrier then orders the writes before the reads.
    if (!wave_active) return;  // the whole workgroup shares this predicate
    constexpr int kGroups = kOutTiles * 4 + 1;         // acc groups + (m, l)
    static_assert(kGroups * 64 * 4 * 4 <= kStageElems * 2, "the merge slots fit in a stage");
    float* mb = reinterpret_cast<float*>(lds);
    auto slot = [&](int w, int g) { return mb + w * (kStageElems / 2) + (g * 64 + lane) * 4; };
#pragma unroll
    for (int mt = 0; mt < kOutTiles; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // groups past output row D are never read (for D = 72, tile 2's
        // group 1 holds the row sum)
        if (32 * mt + 8 * g > D) continue;
        const f32x4 v = {acc[mt][4 * g], acc[mt][4 * g + 1], acc[mt][4 * g + 2], acc[mt][4 * g + 3]};
        *reinterpret_cast<f32x4*>(slot(wave, mt * 4 + g)) = v;
      }
    {
      const f32x4 v = {m_run, l_run, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(slot(wave, kOutTiles * 4)) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // wave w finalizes register group w of every output tile
    // (single-float reads: the loads are independent and all in flight at once)
    float mw[4], lw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* ml = slot(w, kOutTiles * 4);
      mw[w] = ml[0];
      if constexpr (kOnesRow) {
        // the row sum is output row D: tile 2, register 4, lanes with half 0
        lw[w] = mb[w * (kStageElems / 2) + (9 * 64 + col) * 4];
      } else {
        lw[w] = ml[1] + mb[w * (kStageElems / 2) + (kOutTiles * 4 * 64 + (lane ^ 32)) * 4 + 1];
      }
    }
    const float mstar = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    float sc[4], l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc[w] = fast_exp2(mw[w] - mstar);  // 0 for waves without a tile (m = -inf)
      l += sc[w] * lw[w];
    }
    const float inv = 1.0f / l;
    if (qi < N) {
      uint16_t* orow = a.o + b * a.o_sb + h * a.o_sh + static_cast<int64_t>(qi) * a.o_st;
#pragma unroll
      for (int mt = 0; mt < kOutTiles; ++mt) {
        const int d0 = 32 * mt + 8 * wave + 4 * half;
        if (d0 < D) {
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < 4; ++w) o += sc[w] * *reinterpret_cast<const f32x4*>(slot(w, mt * 4 + wave));
          u32x2 st;
          st[0] = pack2<kF16>(o[0] * inv, o[1] * inv);
          st[1] = pack2<kF16>(o[2] * inv, o[3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = st;
        }
      }
    }
    return;
  }

  // ---- prologue: fetch stream tiles 0..2 and wait for tiles 0 and 1.
  // Keys past N in an item's last tile hold copies of key N-1 (see
  // fetch_tile_at), which leave every row max unchanged; only their weights
  // are zeroed.
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) fetch_next();
  wait_fetch_and_sync(after(1, f_s - 1));
  write_ones(0);

  int g0 = 0;  // stream index of the current item's tile 0
  for (int m = 0; m < nitems; ++m, g0 += ntiles) {
    if (m > 0) {
      b = nb;
      h = nh;
      qb = nqb;
      q0 = first_query(qb);
      qi = q0 + col;
      wave_active = q0 < N;
      sign_q(qf, qt);  // loaded during the previous item's last step
#pragma unroll
      for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
      m_run = -__builtin_inff();
      l_run = 0.f;
    }
    if (m + 1 < nitems) coords(item_at(m + 1), nb, nh, nqb);
    // S_0 of the item and its row max in registers (stream tile g0 landed
    // before the last barrier)
    if (wave_active) {
      qk_plain(lds + stage_of(g0) * kStageElems, sa);
      mx = rowmax(sa);
    }
    int j = 0;
    // steady pairs: step j fetches tile j + 3 of this item, which is then
    // neither its last tile (so it is full) nor followed by the switch to the
    // next item's tiles, for every j < ntiles - 4
    const int steady_end = ntiles - 4;
    for (; j + 1 < steady_end; j += 2) {
      step(j, g0 + j, sa, sb, True{}, False{}, False{}, True{});
      step(j + 1, g0 + j + 1, sb, sa, True{}, False{}, False{}, True{});
    }
    for (; j + 2 < ntiles; j += 2) {
      step(j, g0 + j, sa, sb, True{}, False{}, False{}, False{});
      step(j + 1, g0 + j + 1, sb, sa, True{}, False{}, False{}, False{});
    }
    if (j + 1 < ntiles) {
      step(j, g0 + j, sa, sb, True{}, False{}, False{}, False{});
      if (half_tail) step(j + 1, g0 + j + 1, sb, sa, False{}, True{}, True{}, False{});
      else if (ragged) step(j + 1, g0 + j + 1, sb, sa, False{}, True{}, False{}, False{});
      else step(j + 1, g0 + j + 1, sb, sa, False{}, False{}, False{}, False{});
    } else {
      // (an odd tile count or a single tile: this tile's Q K^T ran in the
      // loop or before it)
      if (half_tail) step(j, g0 + j, sa, sb, False{}, True{}, True{}, False{});
      else if (ragged) step(j, g0 + j, sa, sb, False{}, True{}, False{}, False{});
      else step(j, g0 + j, sa, sb, False{}, False{}, False{}, False{});
    }

    // ---- epilogue: O = acc / l in bf16, rows < N only.  The tile goes
    // through the LDS stage of the item's last key tile (free until the next
    // step refills it), so that each global store writes 16 contiguous bytes
    // of a row and consecutive lanes write consecutive bytes of the rows.
    {
      constexpr int kOS = 72;  // row stride of the staged tile (elements)
      static_assert(NW * 32 * kOS <= kStageElems, "staged output tile must fit in a stage");
      uint16_t* ob = lds + stage_of(g0 + ntiles - 1) * kStageElems + wave * 32 * kOS;
      if (wave_active) {
        float l;
        if constexpr (kOnesRow) {
          // row D sits in output tile 2, register 4, of the lanes with half == 0
          l = lower_half_value(acc[2][4]);
        } else {
          l = sum_across_halves(l_run);
        }
        const float inv = 1.0f / l;
#pragma unroll
        for (int mt = 0; mt < kOutTiles; ++mt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * mt + 8 * g + 4 * half;
            if (d0 < D) {
              u32x2 w;
              w[0] = pack2<kF16>(acc[mt][4 * g + 0] * inv, acc[mt][4 * g + 1] * inv);
              w[1] = pack2<kF16>(acc[mt][4 * g + 2] * inv, acc[mt][4 * g + 3] * inv);
              *reinterpret_cast<u32x2*>(ob + col * kOS + d0) = w;
            }
          }
        // store k covers rows kRows*k .. kRows*k + kRows-1: lane l writes
        // 16-byte chunk l % (D/8) of row kRows*k + l / (D/8).  Ordinary
        // (write-back) stores: the next kernel of an encoder block, the output
        // projection, reads this output at once and finds it in the caches.
        // Non-temporal stores made this call about 4% faster on its own but
        // the projection after it slower by more (384 px: the pair took 328
        // against 316 us).
        constexpr int kRowChunks = D / 8, kRows = 64 / kRowChunks;
        const int r0 = lane / kRowChunks, ch = lane - r0 * kRowChunks;
        const uint16_t* src = ob + r0 * kOS + 8 * ch;
        uint16_t* dst = a.o + b * a.o_sb + h * a.o_sh + static_cast<int64_t>(q0 + r0) * a.o_st + 8 * ch;
        const int64_t dst_step = static_cast<int64_t>(kRows) * a.o_st;
#pragma unroll
        for (int k = 0; k < (32 + kRows - 1) / kRows; ++k) {
          const int row = kRows * k + r0;
          if (r0 < kRows && row < 32 && q0 + row < N)
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src + kRows * k * kOS);
          dst += dst_step;
        }
      }
      // every wave is done with the stage before the next step refills it
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
}

template <int D, int NW, bool kSplit, bool kF16, bool kMulti = false>
int launch(const KernelArgs& ka, hipStream_t stream) {
  int qblocks = ka.qblocks, H = ka.H;
  if constexpr (kSplit) {
    // the split kernel divides by qblocks and H with multipliers packed
    // above them: exact while items * qblocks <= 2^16 and pairs * H <= 2^20,
    // and the products item * mq and pair * mh must fit in 32 bits (the
    // launcher picks the split path only within these bounds)
    if (ka.qblocks < 1 || ka.qblocks > 255 || H < 1 || H > 2047) return VITATTN_ERR_LAUNCH;
    const int64_t pairs = ka.items / ka.qblocks;
    const int64_t mq = ((int64_t(1) << 16) + ka.qblocks - 1) / ka.qblocks;
    const int64_t mh = ((int64_t(1) << 20) + H - 1) / H;
    if (static_cast<int64_t>(ka.items) * ka.qblocks > (int64_t(1) << 16) || pairs * H > (int64_t(1) << 20) ||
        ka.items * mq >= (int64_t(1) << 32) || pairs * mh >= (int64_t(1) << 32))
      return VITATTN_ERR_LAUNCH;
    qblocks = static_cast<int>(static_cast<uint32_t>(ka.qblocks) | (static_cast<uint32_t>(mq) << 8));
    H = static_cast<int>(static_cast<uint32_t>(H) | (static_cast<uint32_t>(mh) << 11));
  }
  hipLaunchKernelGGL((fwd_kernel<D, NW, kSplit, kF16, kMulti>), dim3(ka.grid), dim3(64 * NW), 0, stream, ka.grid,
                     qblocks, H, ka.N, ka.i_st, ka.qsign ? -ka.c : ka.c, ka.q, ka.k, ka.v, ka.o, ka.items);
  return hipGetLastError() == hipSuccess ? VITATTN_OK : VITATTN_ERR_LAUNCH;
}

}  // namespace

int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  // several host threads may launch at once: the cache entries are atomic
  static std::atomic<int> cache[64];
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

template <bool kF16>
int launch_typed(const KernelArgs& ka, int D, const FwdShape& sh, hipStream_t s) {
  // split keys over more than 4 key tiles: waves loop over their tiles
  const bool multi = ka.N > 4 * kBlockN;
  if (D == 64) {
    if (sh.split) return multi ? launch<64, 4, true, kF16, true>(ka, s) : launch<64, 4, true, kF16>(ka, s);
    if (sh.waves == 4) return launch<64, 4, false, kF16>(ka, s);
    if (sh.waves == 2) return launch<64, 2, false, kF16>(ka, s);
    return launch<64, 1, false, kF16>(ka, s);
  }
  if (sh.split) return multi ? launch<72, 4, true, kF16, true>(ka, s) : launch<72, 4, true, kF16>(ka, s);
  if (sh.waves == 4) return launch<72, 4, false, kF16>(ka, s);
  if (sh.waves == 2) return launch<72, 2, false, kF16>(ka, s);
  return launch<72, 1, false, kF16>(ka, s);
}

}  // namespace

int launch_fwd(const FwdArgs& f, void* stream) {
  KernelArgs ka{};
  ka.q = f.q;
  ka.k = f.k;
  ka.v = f.v;
  ka.o = f.o;
  // Q, K and V share strides in both layouts, and a 64-token tile spans
  // less than 2 GiB (both checked by the caller)
  if (f.k_sb != f.q_sb || f.v_sb != f.q_sb || f.k_sh != f.q_sh || f.v_sh != f.q_sh ||
      f.k_st != f.q_st || f.v_st != f.q_st || 64 * f.q_st >= (int64_t(1) << 30) ||
      64 * f.o_st >= (int64_t(1) << 30))
    return VITATTN_ERR_LAUNCH;
  {
    // the kernel derives every stride from the layout (contiguous tensors)
    const int64_t nd = static_cast<int64_t>(f.N) * f.D, hd = static_cast<int64_t>(f.H) * f.D;
    const bool sep = f.q_st == f.D;
    const bool ok = sep ? (f.q_sh == nd && f.q_sb == f.H * nd && f.o_st == f.D && f.o_sh == nd &&
                           f.o_sb == f.H * nd)
                        : (f.q_st == 3 * hd && f.q_sh == f.D && f.q_sb == f.N * 3 * hd &&
                           f.o_st == hd && f.o_sh == f.D && f.o_sb == f.N * hd);
    if (!ok) return VITATTN_ERR_LAUNCH;
  }
  ka.i_sb = f.q_sb;
  ka.i_sh = f.q_sh;
  ka.i_st = static_cast<int>(f.q_st);
  ka.o_sb = f.o_sb;
  ka.o_sh = f.o_sh;
  ka.o_st = static_cast<int>(f.o_st);
  ka.H = f.H;
  ka.N = f.N;
  // A zero scale would turn masked (-inf) logits into NaN; any scale below
  // 1e-30 gives weights exp2(~1e-28) == 1 either way.
  const float abs_scale = f.scale < 0.f ? -f.scale : f.scale;
  ka.c = (abs_scale > 1e-30f ? abs_scale : 1e-30f) * kLog2e;
  ka.qsign = f.scale < 0.f ? 0x80008000u : 0u;
  const FwdShape sh = fwd_shape(f.B, f.H, f.N, compute_units());
  ka.qblocks = sh.qblocks;
  ka.items = sh.items;
  ka.grid = sh.grid;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return f.f16 ? launch_typed<true>(ka, f.D, sh, s) : launch_typed<false>(ka, f.D, sh, s);
}

}  // namespace vitattn
