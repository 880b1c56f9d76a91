// The linear layers around the attention of a ViT block on gfx950:
//
//   out[m][n] = sum_k x[m][k] * w[n][k] + bias[n] (+ residual[m][n])
//
// x is [M][K] (tokens x features, row-major), w is [Nout][K] (the layer's
// weight as stored: output features x input features), all 16-bit (bf16 or
// fp16), fp32 accumulation, one rounding of the final sum to the output
// format.  Two uses on the pages: the block's fused qkv projection, whose
// [M][3*H*D] output is the packed [B][N][3][H][D] buffer the attention reads
// (FluxVLA "Inference acceleration" section 1 fuses it as matmul_rope_qkv;
// ViT needs no rotary embedding), and the output projection with its bias
// and the residual add fused into the epilogue (same page, section 3,
// matmul_bias_res).
//
// Work decomposition
//   * one workgroup per BM x BN output tile; WM x WN waves, each owning a
//     TM x TN sub-tile as (TN/32) x (TM/32) accumulators of the 32x32 MFMA
//     (256 x 256, 128 x 128 or 64 x 128 tiles, the largest that still give
//     one workgroup per compute unit);
//   * the product is formed transposed, C^T = W X^T (every lane holds runs
//     of four consecutive output features of one token); the epilogue
//     stages 32-token slabs through LDS as fp32 and writes whole 128-byte
//     row segments, adding bias and residual on the way;
//   * k in tiles of 32: x rows and w rows go direct to LDS (128-bit
//     global_load_lds, no staging registers) into a four-stage ring, three
//     tiles ahead, one barrier per tile, waited for two tiles ahead.  An LDS row holds the tile's 64
//     bytes of one x or w row as four 16-byte chunks, chunk c of row r at
//     position c ^ ((r >> 2) & 3): sixteen consecutive rows read at one
//     chunk then fall in sixteen distinct bank groups, with no padding;
//   * operand reads for the next k step are issued before the MFMAs of the
//     current one, and those of the next tile's first step before the
//     barrier that ends a tile (its data was published one barrier earlier);
//   * rows past M (or Nout) load row M-1 (Nout-1) and are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitattn_internal.h"

namespace vitattn {
namespace {

typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 lf16x8 __attribute__((ext_vector_type(8)));
typedef float lf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t lu32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;         // k per tile
constexpr int kRowElems = 32;   // LDS row stride in elements (64 bytes)
constexpr int kSlotsRow = 4;    // 16-byte LDS slots per row
constexpr int kStagesL = 4;

struct LinearArgs {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* bias;      // may be NULL
  const uint16_t* residual;  // may be NULL
  uint16_t* out;
  int M, K, Nout;
  int mblocks, nblocks;
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved: the clobber is intended
// One direct-to-LDS fetch: each lane copies 16 bytes from g + off into slot
// `lane` of the 64 x 16-byte block at LDS byte address lds_addr (M0).  The
// kernel orders these itself (vmcnt waits and a barrier before a stage is
// read; a stage is refilled only after the barrier that ends its reads).
__device__ __forceinline__ void ldma16(const char* g, uint32_t off, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off), "s"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <bool kF16>
__device__ __forceinline__ lf32x16 lmma(lbf16x8 a, lbf16x8 b, lf32x16 c) {
  if constexpr (kF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(lf16x8, a), __builtin_bit_cast(lf16x8, b),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool kF16>
__device__ __forceinline__ float widen16(uint32_t bits16) {
  if constexpr (kF16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  } else {
    return __builtin_bit_cast(float, bits16 << 16);
  }
}

template <bool kF16>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) {
  if constexpr (kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 p;
    p[0] = static_cast<_Float16>(lo);
    p[1] = static_cast<_Float16>(hi);
    return __builtin_bit_cast(uint32_t, p);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 p;
    p[0] = static_cast<__bf16>(lo);
    p[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, p);
  }
}

__device__ __forceinline__ int lxcd_remap(int bid, int grid) {
  const int q = grid >> 3, r = grid & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + (x < r ? x : r) + i;
}

// kStream: the output goes out with non-temporal stores (see launch_linear_typed)
template <int WM, int WN, int TM, int TN, bool kF16, bool kStream>
__global__ __launch_bounds__(64 * WM * WN) void linear_kernel(LinearArgs a) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM, BN = WN * TN;
  constexpr int kRows = BM + BN;                    // x rows then w rows in a stage
  constexpr int kStageElems = kRows * kRowElems;
  constexpr int kInstr = kRows * kSlotsRow / 64;    // fetch instructions per stage
  static_assert(kRows * kSlotsRow % 64 == 0, "whole fetch instructions");
  constexpr int kInstrX = BM * kSlotsRow / 64;      // the first kInstrX fetch x rows
  static_assert(BM * kSlotsRow % 64 == 0, "no fetch instruction mixes x and w rows");
  constexpr int kPerWave = (kInstr + NW - 1) / NW;
  constexpr int kMinPerWave = kInstr / NW;
  constexpr int FM = TM / 32, FN = TN / 32;         // accumulator blocks per wave
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStagesL * kStageElems];
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)lds));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int col = lane & 31, half = lane >> 5;

  // Tile order: each XCD takes a contiguous range of tiles (lxcd_remap),
  // and within it tiles run in groups of kGroupM token blocks, output
  // feature blocks slowest inside a group, so the workgroups resident in an
  // XCD at one time share both x and w rows in its L2.
  constexpr int kGroupM = 8;
  const int tile = lxcd_remap(blockIdx.x, gridDim.x);
  const int per_group = kGroupM * a.nblocks;
  const int first_m = (tile / per_group) * kGroupM;
  const int gsize = a.mblocks - first_m < kGroupM ? a.mblocks - first_m : kGroupM;
  const int within = tile - (tile / per_group) * per_group;
  const int mb = first_m + within % gsize, nb = within / gsize;
  const int m0 = mb * BM, n0 = nb * BN;
  const int M = a.M, K = a.K, Nout = a.Nout;
  const int ktiles = K / kBK;

  // this lane's 16-byte source chunk in fetch instruction i of this wave:
  // slot s = I*64 + lane of the stage is position s % 4 of row s / 4, which
  // holds chunk (s % 4) ^ ((row >> 2) & 3); rows < BM are x rows m0.., the
  // rest w rows n0..
  const char* xg = reinterpret_cast<const char*>(a.x);
  const char* wg = reinterpret_cast<const char*>(a.w);
  uint32_t f_off[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int I = i * NW + wave;
    const int s = I * 64 + lane;
    const int row = s / kSlotsRow;
    const int c = (s - row * kSlotsRow) ^ ((row >> 2) & 3);
    int r;
    if (row < BM) {
      r = m0 + row;
      r = r < M ? r : M - 1;
    } else {
      r = n0 + row - BM;
      r = r < Nout ? r : Nout - 1;
    }
    f_off[i] = static_cast<uint32_t>((static_cast<int64_t>(r) * K + c * 8) * 2);
  }
  // f_off is a byte offset below 2^32: the host limits M*K and Nout*K
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = lds_base + 2 * (t % kStagesL) * kStageElems;
    const uint32_t koff = static_cast<uint32_t>(t * kBK * 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int I = i * NW + wave;
      if (i >= kMinPerWave && I >= kInstr) continue;
      ldma16(I < kInstrX ? xg : wg, f_off[i] + koff, stage + 2 * I * 512);
    }
  };
  auto wait_and_sync = [&](int tiles_in_flight) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
#define VITATTN_LWAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
    if (tiles_in_flight == 0) {
      VITATTN_LWAIT(0);
    } else if (tiles_in_flight == 1) {
      VITATTN_LWAIT(kMinPerWave);
    } else {
      VITATTN_LWAIT(2 * kMinPerWave);
    }
#undef VITATTN_LWAIT
    asm volatile("s_barrier" ::: "memory");
  };

  lf32x16 acc[FN][FM];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // operand rows: A (w) rows BM + wn*TN + 32j + col, B (x) rows
  // wm*TM + 32i + col, both at k chunk 2*ks + half of the tile; the row bits
  // that pick the chunk position are those of col (32j, 32i and the bases
  // are multiples of 32)
  const int swz = (col >> 2) & 3;
  const int a_row = (BM + wn * TN + col) * kRowElems, b_row = (wm * TM + col) * kRowElems;
  const int c_off0 = 8 * ((0 + half) ^ swz), c_off1 = 8 * ((2 + half) ^ swz);

  // operands of one k step (ks = 0, 1) of the tile in stage `st`
  auto load_ops = [&](const uint16_t* st, int ks, lbf16x8* av, lbf16x8* bv) __attribute__((always_inline)) {
    const int co = ks ? c_off1 : c_off0;
#pragma unroll
    for (int j = 0; j < FN; ++j) av[j] = *reinterpret_cast<const lbf16x8*>(st + a_row + 32 * j * kRowElems + co);
#pragma unroll
    for (int i = 0; i < FM; ++i) bv[i] = *reinterpret_cast<const lbf16x8*>(st + b_row + 32 * i * kRowElems + co);
  };
  // tiles fetched after tile t (0 .. kStagesL-2) when the fetch of tile
  // `last` is the most recent
  auto in_flight_after = [&](int t, int last) { return last > t ? last - t : 0; };

  // Schedule: the fetch of tile t+3 is issued at the top of tile t; at the
  // end of tile t each wave waits for its part of tile t+2, reads the first
  // k step of tile t+1 (complete and visible since the previous barrier)
  // and meets the others.  The barrier both publishes tile t+2 and frees
  // stage t for the fetch of tile t+4.
  const int pre = ktiles < kStagesL - 1 ? ktiles : kStagesL - 1;
  for (int t = 0; t < pre; ++t) fetch(t);
  wait_and_sync(in_flight_after(1, pre - 1));  // tiles 0 and 1 landed
  lbf16x8 a0[FN], b0[FM], a1[FN], b1[FM];
  load_ops(lds, 0, a0, b0);
  for (int t = 0; t < ktiles; ++t) {
    if (t + kStagesL - 1 < ktiles) fetch(t + kStagesL - 1);
    const uint16_t* st = lds + (t % kStagesL) * kStageElems;
    load_ops(st, 1, a1, b1);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[j][i] = lmma<kF16>(a0[j], b0[i], acc[j][i]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[j][i] = lmma<kF16>(a1[j], b1[i], acc[j][i]);
    if (t + 1 < ktiles) {
      const int last = t + kStagesL - 1 < ktiles ? t + kStagesL - 1 : ktiles - 1;
      asm volatile("" ::: "memory");
#define VITATTN_LWAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
      if (in_flight_after(t + 2, last) == 0) {
        VITATTN_LWAIT(0);
      } else {
        VITATTN_LWAIT(kMinPerWave);
      }
#undef VITATTN_LWAIT
      load_ops(lds + ((t + 1) % kStagesL) * kStageElems, 0, a0, b0);
      asm volatile("s_barrier" ::: "memory");
    }
  }

  // ---- epilogue.  acc[j][i][r] is C^T for output feature
  // n0 + wn*TN + 32j + 8*(r/4) + 4*half + (r%4) and token m0 + wm*TM + 32i +
  // col.  Each 32-token slab i of the wave's tile goes through the wave's
  // own LDS region as fp32 (the ring is free once every wave has left the
  // loop), and comes back as rows: lane l then holds 8 consecutive features
  // of one token, adds bias and residual and writes 16 bytes, TN/8 lanes
  // covering one row segment of the tile (128 bytes for TN = 64).
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int kSlabStride = TN + 4;  // floats per staged row (272 bytes for TN = 64)
  static_assert(NW * 32 * kSlabStride * 4 <= kStagesL * kStageElems * 2, "staging fits in the ring");
  constexpr int kLanesRow = TN / 8, kRowsRead = 64 / kLanesRow;  // read-back: lanes per row, rows per pass
  static_assert(TN % 8 == 0 && 32 % kRowsRead == 0, "whole rows per read-back pass");
  float* slab = reinterpret_cast<float*>(lds) + wave * 32 * kSlabStride;
  const int rrow = lane / kLanesRow, rch = lane % kLanesRow;  // row within the pass, 8-feature chunk
  const int n = n0 + wn * TN + 8 * rch;
  float bsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) bsum[e] = 0.f;
  if (a.bias && n < Nout) {
    const uint4 bb = *reinterpret_cast<const uint4*>(a.bias + n);
    const uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bsum[2 * e] = widen16<kF16>(bw[e] & 0xffffu);
      bsum[2 * e + 1] = widen16<kF16>(bw[e] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = {acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]};
        *reinterpret_cast<float4*>(slab + col * kSlabStride + 32 * j + 8 * g + 4 * half) = v;
      }
#pragma unroll
    for (int q = 0; q < 32 / kRowsRead; ++q) {
      const int row = kRowsRead * q + rrow;
      const float4 lo = *reinterpret_cast<const float4*>(slab + row * kSlabStride + 8 * rch);
      const float4 hi = *reinterpret_cast<const float4*>(slab + row * kSlabStride + 8 * rch + 4);
      const int m = m0 + wm * TM + 32 * i + row;
      if (m >= M || n >= Nout) continue;
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += bsum[e];
      const int64_t o = static_cast<int64_t>(m) * Nout + n;
      if (a.residual) {
        const uint4 rr = *reinterpret_cast<const uint4*>(a.residual + o);
        const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] += widen16<kF16>(rw[e] & 0xffffu);
          v[2 * e + 1] += widen16<kF16>(rw[e] >> 16);
        }
      }
      uint4 w;
      w.x = pack16x2<kF16>(v[0], v[1]);
      w.y = pack16x2<kF16>(v[2], v[3]);
      w.z = pack16x2<kF16>(v[4], v[5]);
      w.w = pack16x2<kF16>(v[6], v[7]);
      const lu32x4 wv = {w.x, w.y, w.z, w.w};
      if constexpr (kStream)
        __builtin_nontemporal_store(wv, reinterpret_cast<lu32x4*>(a.out + o));
      else
        *reinterpret_cast<lu32x4*>(a.out + o) = wv;
    }
  }
}

template <int WM, int WN, int TM, int TN, bool kF16, bool kStream = false>
int launch_linear_cfg(const LinearArgs& la0, hipStream_t s) {
  LinearArgs la = la0;
  constexpr int BM = WM * TM, BN = WN * TN;
  la.mblocks = (la.M + BM - 1) / BM;
  la.nblocks = (la.Nout + BN - 1) / BN;
  const int64_t grid = static_cast<int64_t>(la.mblocks) * la.nblocks;
  hipLaunchKernelGGL((linear_kernel<WM, WN, TM, TN, kF16, kStream>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WM * WN), 0, s, la);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

template <bool kF16>
int launch_linear_typed(const LinearArgs& la, hipStream_t s) {
  // the largest tiles that still give a workgroup per compute unit (256 on
  // MI355X): 256 x 256 (eight waves of 128 x 64), 128 x 128 (four waves of
  // 64 x 64); below that, 64 x 64 tiles (four waves of 32 x 32) while they
  // number at most 448, else 64 x 128 (four waves of 32 x 64).  (On the
  // 224 px projections, M = 512: 64 x 64 tiles take the output projection
  // from 10.0 to 8.4 us and the qkv projection from 10.2 to 9.7 us; past
  // about 1.75 tiles per compute unit the 64 x 128 tiles are faster.)
  auto tiles = [&](int bm, int bn) {
    return static_cast<int64_t>((la.M + bm - 1) / bm) * ((la.Nout + bn - 1) / bn);
  };
  if (tiles(256, 256) >= 256) {
    // Outputs larger than half the 256 MB last-level cache go out with
    // non-temporal stores: such an output cannot stay cached for the next
    // kernel anyway, and streamed past the L2 it leaves that cache to the x
    // and w rows other tiles still read (qkv projection at 384 px x 48,
    // 242 MB: 322 against 330 us on its own, and with the attention call
    // that reads it 481 against 487 us for the pair).  Smaller outputs use
    // write-back stores, where the next kernel finds them (non-temporal
    // stores gained nothing for the 80 MB output projection).  The smaller
    // tiles below only serve outputs under 256 x 65536 elements.
    if (static_cast<int64_t>(la.M) * la.Nout * 2 > (int64_t(128) << 20))
      return launch_linear_cfg<2, 4, 128, 64, kF16, true>(la, s);
    return launch_linear_cfg<2, 4, 128, 64, kF16>(la, s);
  }
  if (tiles(128, 128) >= 256) return launch_linear_cfg<2, 2, 64, 64, kF16>(la, s);
  if (tiles(64, 64) <= 448) return launch_linear_cfg<2, 2, 32, 32, kF16>(la, s);
  return launch_linear_cfg<2, 2, 32, 64, kF16>(la, s);
}

}  // namespace

int launch_linear(const LinearCall& c, void* stream) {
  LinearArgs la{};
  la.x = c.x;
  la.w = c.w;
  la.bias = c.bias;
  la.residual = c.residual;
  la.out = c.out;
  la.M = c.M;
  la.K = c.K;
  la.Nout = c.Nout;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return c.f16 ? launch_linear_typed<true>(la, s) : launch_linear_typed<false>(la, s);
}

}  // namespace vitattn
