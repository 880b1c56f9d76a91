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
//     TM x TN sub-tile as (TN/32) x (TM/32) accumulators of the 32x32 MFMA;
//   * the product is formed transposed, C^T = W X^T, so that every lane
//     holds four consecutive output features of one token: the epilogue then
//     reads bias and residual and writes the output 8 bytes at a time;
//   * k in tiles of 32: x rows and w rows go direct to LDS (128-bit
//     global_load_lds, no staging registers) into a three-stage ring, two
//     tiles ahead, one barrier per tile.  LDS rows are 80 bytes (64 of data
//     and a 16-byte slot that receives a copy and is never read): sixteen
//     consecutive rows then fall in disjoint banks for the 128-bit operand
//     reads;
//   * rows past M (or Nout) load row M-1 (Nout-1) and are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitattn_internal.h"

namespace vitattn {
namespace {

typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 lf16x8 __attribute__((ext_vector_type(8)));
typedef float lf32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t lu32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 32;         // k per tile
constexpr int kRowElems = 40;   // LDS row stride in elements (80 bytes)
constexpr int kSlotsRow = 5;    // 16-byte LDS slots per row (4 of data)
constexpr int kStagesL = 3;

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

template <int WM, int WN, int TM, int TN, bool kF16>
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

  const int tile = lxcd_remap(blockIdx.x, gridDim.x);
  const int mb = tile / a.nblocks, nb = tile - mb * a.nblocks;
  const int m0 = mb * BM, n0 = nb * BN;
  const int M = a.M, K = a.K, Nout = a.Nout;
  const int ktiles = K / kBK;

  // this lane's 16-byte source chunk in fetch instruction i of this wave:
  // slot s = I*64 + lane of the stage holds row s / 5, chunk s % 5 (chunk 4
  // repeats chunk 3); rows < BM are x rows m0.., the rest w rows n0..
  const char* xg = reinterpret_cast<const char*>(a.x);
  const char* wg = reinterpret_cast<const char*>(a.w);
  uint32_t f_off[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int I = i * NW + wave;
    const int s = I * 64 + lane;
    const int row = s / kSlotsRow;
    int c = s - row * kSlotsRow;
    c = c < 4 ? c : 3;
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
    } else {
      VITATTN_LWAIT(kMinPerWave);
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

  // operand rows: A (w) rows wn*TN + 32j + col, B (x) rows wm*TM + 32i + col;
  // k offset 8*half (+16 for the second k step)
  const int a_off = (BM + wn * TN + col) * kRowElems + 8 * half;
  const int b_off = (wm * TM + col) * kRowElems + 8 * half;

  fetch(0);
  if (ktiles > 1) fetch(1);
  wait_and_sync(ktiles > 1 ? 1 : 0);
  for (int t = 0; t < ktiles; ++t) {
    if (t + 2 < ktiles) fetch(t + 2);
    const uint16_t* st = lds + (t % kStagesL) * kStageElems;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      lbf16x8 av[FN], bv[FM];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        av[j] = *reinterpret_cast<const lbf16x8*>(st + a_off + 32 * j * kRowElems + 16 * ks);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        bv[i] = *reinterpret_cast<const lbf16x8*>(st + b_off + 32 * i * kRowElems + 16 * ks);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = lmma<kF16>(av[j], bv[i], acc[j][i]);
    }
    // tile t+1 must have landed (t+2 may stay in flight) and every wave must
    // be done with stage t before it is refilled with tile t+3
    if (t + 1 < ktiles) wait_and_sync(t + 2 < ktiles ? 1 : 0);
  }

  // ---- epilogue.  acc[j][i] is C^T for output features n0 + wn*TN + 32j +
  // 8*(r/4) + 4*half + (r%4) and token m0 + wm*TM + 32i + col: each lane
  // holds, per group g = r/4, four consecutive features of one token.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * TN + 32 * j + 8 * g + 4 * half;
      if (n >= Nout) continue;  // Nout is a multiple of 8: all four or none
      float bsum[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.bias) {
        const lu32x2 bb = *reinterpret_cast<const lu32x2*>(a.bias + n);
        bsum[0] = widen16<kF16>(bb[0] & 0xffffu);
        bsum[1] = widen16<kF16>(bb[0] >> 16);
        bsum[2] = widen16<kF16>(bb[1] & 0xffffu);
        bsum[3] = widen16<kF16>(bb[1] >> 16);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + 32 * i + col;
        if (m >= M) continue;
        const int64_t o = static_cast<int64_t>(m) * Nout + n;
        float v0 = acc[j][i][4 * g + 0] + bsum[0];
        float v1 = acc[j][i][4 * g + 1] + bsum[1];
        float v2 = acc[j][i][4 * g + 2] + bsum[2];
        float v3 = acc[j][i][4 * g + 3] + bsum[3];
        if (a.residual) {
          const lu32x2 rr = *reinterpret_cast<const lu32x2*>(a.residual + o);
          v0 += widen16<kF16>(rr[0] & 0xffffu);
          v1 += widen16<kF16>(rr[0] >> 16);
          v2 += widen16<kF16>(rr[1] & 0xffffu);
          v3 += widen16<kF16>(rr[1] >> 16);
        }
        lu32x2 w;
        w[0] = pack16x2<kF16>(v0, v1);
        w[1] = pack16x2<kF16>(v2, v3);
        *reinterpret_cast<lu32x2*>(a.out + o) = w;
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, bool kF16>
int launch_linear_cfg(const LinearArgs& la0, hipStream_t s) {
  LinearArgs la = la0;
  constexpr int BM = WM * TM, BN = WN * TN;
  la.mblocks = (la.M + BM - 1) / BM;
  la.nblocks = (la.Nout + BN - 1) / BN;
  const int64_t grid = static_cast<int64_t>(la.mblocks) * la.nblocks;
  hipLaunchKernelGGL((linear_kernel<WM, WN, TM, TN, kF16>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WM * WN), 0, s, la);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

template <bool kF16>
int launch_linear_typed(const LinearArgs& la, hipStream_t s) {
  // 256 x 256 tiles (eight waves of 128 x 64) when they still give a few
  // hundred workgroups; 128 x 128 tiles (four waves of 64 x 64) otherwise
  const int64_t big = static_cast<int64_t>((la.M + 255) / 256) * ((la.Nout + 255) / 256);
  if (big >= 256) return launch_linear_cfg<2, 4, 128, 64, kF16>(la, s);
  return launch_linear_cfg<2, 2, 64, 64, kF16>(la, s);
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
