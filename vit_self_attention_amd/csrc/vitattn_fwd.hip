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
//   * one workgroup per (image, head, block of 32*NW queries); NW waves of
//     64 lanes, each wave owning 32 queries;
//   * keys in tiles of 64, loaded cooperatively from HBM with 128-bit loads
//     and double-buffered in LDS: K row-major, V transposed (V^T) so both
//     matrix products read their operands with contiguous LDS loads;
//   * both products on bf16 MFMA with fp32 accumulation, in transposed form:
//       S^T = K Q^T       (v_mfma_f32_32x32x16_bf16; D = 72 adds one 32x32x8)
//       O^T += V^T P^T    (v_mfma_f32_32x32x16_bf16)
//     With S^T in the accumulator layout, lane l holds 16 keys of query
//     (l mod 32) per 32x32 block: the row max and row sum are mostly
//     in-lane, and the accumulator registers are, after conversion to bf16,
//     exactly the B operand of the second product (keys permuted within each
//     group of 16, matched by the order in which V^T is read);
//   * online softmax in base 2: m = running max of scale*log2(e)*s,
//     p = exp2(scale*log2(e)*s - m), rescale by exp2(m_old - m_new);
//   * D = 72: the P V product runs three 32-row output tiles (d 0..95); the
//     spare row d = 72 multiplies P by a row of ones, which yields the
//     softmax denominator from the same bf16 probabilities that weight V.
//   * tails: keys >= N are zero-filled in LDS and masked to -inf; queries
//     >= N are computed on zero rows and never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitattn.h"
#include "vitattn_internal.h"

namespace vitattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockN = 64;          // keys per tile
constexpr int kKStride = 72;         // LDS row stride of the K tile (elements): 144 B
constexpr int kVStride = kBlockN + 4;  // LDS row stride of the V^T tile (elements): 136 B
constexpr float kLog2e = 1.4426950408889634f;

struct KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  int64_t v_sb, v_sh, v_st;
  int64_t o_sb, o_sh, o_st;
  int H, N;
  int qblocks;     // query blocks per (image, head)
  int grid;        // total workgroups
  float c;         // |scale| * log2(e)
  uint32_t qsign;  // 0x80008000 when scale < 0: Q is negated instead
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = static_cast<__bf16>(lo);
  p[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, p);
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

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(KernelArgs a) {
  constexpr int kThreads = 64 * NW;
  constexpr int kChunksPerRow = D / 8;                 // 16-byte chunks per row
  constexpr int kChunks = kBlockN * kChunksPerRow;     // chunks per tile
  constexpr int kChunksPerThread = (kChunks + kThreads - 1) / kThreads;
  constexpr bool kOnesRow = (D % 32) != 0;             // spare output row carries the row sum
  constexpr int kOutTiles = kOnesRow ? (D + 32) / 32 : D / 32;  // 3 for D=72, 2 for D=64
  constexpr int kKTile = kBlockN * kKStride;           // elements
  constexpr int kVTile = D * kVStride;                 // elements

  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kVTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query within the wave (MFMA column)
  const int half = lane >> 5;  // which half of the K dimension this lane feeds

  const int tile_id = xcd_remap(blockIdx.x, a.grid);
  const int bh = tile_id / a.qblocks;
  const int qb = tile_id - bh * a.qblocks;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int N = a.N;

  const uint16_t* kbase = a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t* vbase = a.v + b * a.v_sb + h * a.v_sh;

  // ---- this lane's query row as the B operand of S^T = K Q^T
  const int q0 = qb * (32 * NW) + wave * 32;
  const int qi = q0 + col;
  const bool wave_active = q0 < N;
  bf16x8 qf[4];
  bf16x4 qt = {};
  {
    const uint16_t* qrow = a.q + b * a.q_sb + h * a.q_sh + static_cast<int64_t>(qi) * a.q_st;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qi < N) w = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * half);
      w ^= a.qsign;
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
    if constexpr (D == 72) {
      u32x2 w = {0u, 0u};
      if (qi < N) w = *reinterpret_cast<const u32x2*>(qrow + 64 + 4 * half);
      w ^= a.qsign;
      qt = __builtin_bit_cast(bf16x4, w);
    }
  }

  // ---- cooperative tile loads: global -> registers -> LDS
  u32x4 kreg[kChunksPerThread], vreg[kChunksPerThread];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / kChunksPerRow, cc = c - row * kChunksPerRow;
      const int key = kb + row;
      u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
      if (c < kChunks && key < N) {
        kw = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.k_st + cc * 8);
        vw = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * a.v_st + cc * 8);
      }
      kreg[i] = kw;
      vreg[i] = vw;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int c = tid + i * kThreads;
      if (c < kChunks) {
        const int row = c / kChunksPerRow, cc = c - row * kChunksPerRow;
        *reinterpret_cast<u32x4*>(&lds_k[buf][row * kKStride + cc * 8]) = kreg[i];
        uint16_t* vt = &lds_v[buf][(cc * 8) * kVStride + row];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[(2 * e) * kVStride] = static_cast<uint16_t>(vreg[i][e] & 0xffffu);
          vt[(2 * e + 1) * kVStride] = static_cast<uint16_t>(vreg[i][e] >> 16);
        }
      }
    }
  };

  f32x16 acc[kOutTiles];
#pragma unroll
  for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;  // per-lane partial row sum (D = 64 only)
  const float c = a.c;

  const int ntiles = (N + kBlockN - 1) / kBlockN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const int kb = j * kBlockN;
    if (j + 1 < ntiles) load_tile(kb + kBlockN);

    if (wave_active) {
      const uint16_t* kt = lds_k[buf];
      const uint16_t* vt = lds_v[buf];
      // S^T = K Q^T : two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[blk][r] = 0.f;
        const uint16_t* krow = kt + (32 * blk + col) * kKStride;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 16 * st + 8 * half);
          s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s[blk], 0, 0, 0);
        }
        if constexpr (D == 72) {
          bf16x4 ka = *reinterpret_cast<const bf16x4*>(krow + 64 + 4 * half);
          s[blk] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ka, qt, s[blk], 0, 0, 0);
        }
      }
      // s[blk][r] is the logit of key kb + 32*blk + 8*(r/4) + 4*half + (r%4)
      const bool tail = kb + kBlockN > N;
      if (tail) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * blk + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= N) s[blk][r] = -__builtin_inff();
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;

      float psum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[blk][r], c, -m_new));
          if (tail) {
            const int key = kb + 32 * blk + 8 * (r >> 2) + 4 * half + (r & 3);
            p = key < N ? p : 0.f;
          }
          s[blk][r] = p;
          if constexpr (!kOnesRow) psum += p;
        }
      if constexpr (!kOnesRow) l_run = l_run * alpha + psum;
#pragma unroll
      for (int t = 0; t < kOutTiles; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;

      // O^T += V^T P^T over four 16-key steps.  Step t uses keys
      // kb + 16t + {4*half + 0..3, 8 + 4*half + 0..3}, which are
      // s[t/2][8*(t%2) + 0..7] of this lane.
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int blk = t >> 1, r0 = 8 * (t & 1);
        u32x4 pw;
        pw[0] = pack_bf16x2(s[blk][r0 + 0], s[blk][r0 + 1]);
        pw[1] = pack_bf16x2(s[blk][r0 + 2], s[blk][r0 + 3]);
        pw[2] = pack_bf16x2(s[blk][r0 + 4], s[blk][r0 + 5]);
        pw[3] = pack_bf16x2(s[blk][r0 + 6], s[blk][r0 + 7]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int mt = 0; mt < kOutTiles; ++mt) {
          const int d = 32 * mt + col;
          u32x4 vw;
          if (d < D) {
            const uint16_t* vrow = vt + d * kVStride + 16 * t + 4 * half;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
            vw[0] = lo[0];
            vw[1] = lo[1];
            vw[2] = hi[0];
            vw[3] = hi[1];
          } else {
            // rows past D: the row d == D is all ones (row sum), others zero
            const uint32_t one2 = (d == D) ? 0x3f803f80u : 0u;
            vw[0] = one2;
            vw[1] = one2;
            vw[2] = one2;
            vw[3] = one2;
          }
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pb,
                                                           acc[mt], 0, 0, 0);
        }
      }
    }

    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;

  // ---- epilogue: O = acc / l, bf16, rows < N only
  float l;
  if constexpr (kOnesRow) {
    // row D sits in output tile D/32 at register 4*((D%32)/8) + (D%4) of the
    // lanes with half == ((D%8)/4)
    constexpr int kT = D / 32, kR = 4 * ((D % 32) / 8) + (D % 4), kHalf = (D % 8) / 4;
    const float mine = acc[kT][kR];
    const float other = __shfl_xor(mine, 32);
    l = (half == kHalf) ? mine : other;
  } else {
    l = l_run + __shfl_xor(l_run, 32);
  }
  const float inv = 1.0f / l;
  if (qi < N) {
    uint16_t* orow = a.o + b * a.o_sb + h * a.o_sh + static_cast<int64_t>(qi) * a.o_st;
#pragma unroll
    for (int mt = 0; mt < kOutTiles; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * half;
        if (d0 < D) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[mt][4 * g + 0] * inv, acc[mt][4 * g + 1] * inv);
          w[1] = pack_bf16x2(acc[mt][4 * g + 2] * inv, acc[mt][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      }
  }
}

template <int D, int NW>
int launch(const KernelArgs& ka, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_kernel<D, NW>), dim3(ka.grid), dim3(64 * NW), 0, stream, ka);
  return hipGetLastError() == hipSuccess ? VITATTN_OK : VITATTN_ERR_LAUNCH;
}

}  // namespace

int pick_waves(int B, int H, int N) {
  // Largest workgroup (more K/V reuse per LDS tile) that still gives at
  // least two workgroups per compute unit on the 256-CU part.
  const int64_t pairs = static_cast<int64_t>(B) * H;
  for (int nw = 4; nw > 1; nw >>= 1) {
    const int64_t qblocks = (N + 32 * nw - 1) / (32 * nw);
    if (pairs * qblocks >= 512) return nw;
  }
  return 1;
}

int launch_fwd(const FwdArgs& f, void* stream) {
  KernelArgs ka{};
  ka.q = f.q;
  ka.k = f.k;
  ka.v = f.v;
  ka.o = f.o;
  ka.q_sb = f.q_sb; ka.q_sh = f.q_sh; ka.q_st = f.q_st;
  ka.k_sb = f.k_sb; ka.k_sh = f.k_sh; ka.k_st = f.k_st;
  ka.v_sb = f.v_sb; ka.v_sh = f.v_sh; ka.v_st = f.v_st;
  ka.o_sb = f.o_sb; ka.o_sh = f.o_sh; ka.o_st = f.o_st;
  ka.H = f.H;
  ka.N = f.N;
  ka.c = (f.scale < 0.f ? -f.scale : f.scale) * kLog2e;
  ka.qsign = f.scale < 0.f ? 0x80008000u : 0u;
  const int nw = pick_waves(f.B, f.H, f.N);
  ka.qblocks = (f.N + 32 * nw - 1) / (32 * nw);
  ka.grid = f.B * f.H * ka.qblocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (f.D == 64) {
    if (nw == 4) return launch<64, 4>(ka, s);
    if (nw == 2) return launch<64, 2>(ka, s);
    return launch<64, 1>(ka, s);
  }
  if (nw == 4) return launch<72, 4>(ka, s);
  if (nw == 2) return launch<72, 2>(ka, s);
  return launch<72, 1>(ka, s);
}

}  // namespace vitattn
