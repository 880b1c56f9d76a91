/*
 * libvitattn -- forward pass of the bidirectional multi-head self-attention
 * of a ViT / SigLIP vision encoder on AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every image b < B and head h < H, with Q, K, V the
 * N x D bf16 matrices of that (image, head) over the N patch tokens:
 *
 *     O = softmax(scale * Q K^T) V          (softmax along the key axis)
 *
 * This is the attention core that the Pi0 Flash Attention tutorial
 * ("Pi0 VLA deployment: accelerating the vision encoder with Flash
 * Attention", section 1) names as the dominant cost of the vision encoder,
 * and that its section 3.2 swaps for a fused kernel fed by the block's fused
 * qkv projection, with inputs and outputs unchanged.  Every token attends to
 * every token (no mask); no dropout (inference).
 *
 * Numerics: bf16 inputs (or fp16 with VITATTN_DTYPE_FP16), fp32 accumulation
 * and softmax state, probabilities rounded to the input format (nearest
 * even) for the P V product, output in the input format rounded to nearest
 * even.  Inputs must be finite.  The softmax's running maximum is updated
 * lazily (weights up to 2^32 before a rescale, 2^8 for fp16), so the fp32
 * sums stay finite for |V| below about 2^128 / (N * 2^32) (1e26 at
 * N = 729; fp16 values cannot reach the fp16 bound).
 * Results are deterministic: the same inputs give the same output bits.
 *
 * C ABI only: plain pointers and sizes.  The library allocates no device
 * memory of its own and may be called from several host threads at once.
 * vitattn_fwd keeps no state between calls; the only state is held in plan
 * objects (recorded call sequences, below) that the caller creates and
 * destroys.
 */
#ifndef VITATTN_H
#define VITATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Input layouts. */
enum {
  /* q, k, v: three separate bf16 tensors, each [B][H][N][D] (row-major).
   * out: [B][H][N][D]. */
  VITATTN_LAYOUT_SEPARATE_BHND = 0,
  /* qkv_or_q: the fused qkv activation [B][N][3][H][D] (slot 0 = Q,
   * 1 = K, 2 = V), i.e. the [B, N, 3*H*D] output of the qkv projection;
   * k and v must be NULL.  out: [B][N][H][D], i.e. [B, N, H*D], the input
   * of the output projection. */
  VITATTN_LAYOUT_PACKED_BN3HD = 1,
  /* Element format flag, OR-ed into `layout`: the inputs and the output are
   * IEEE fp16 instead of bf16, with the same shapes and strides.  The fp16
   * autocast of the Pi0 latency report (section 3.2) and the fp16 vision
   * encoder of the VLA speed-up article (section 3.2) run the encoder in
   * this format. */
  VITATTN_DTYPE_FP16 = 16
};

/* Status codes (0 = success; negative = error, nothing launched).  The
 * failures the Pi0 Flash Attention tutorial lists for its attention swap
 * (section 5.2 table: tensors on different devices, a missing or mismatched
 * kernel library, a kernel image not built for the device) surface here as
 * codes rather than exceptions: every argument is checked on the host
 * before a launch, and a library without a gfx950 image for the current
 * device returns VITATTN_ERR_LAUNCH. */
enum {
  VITATTN_OK = 0,
  VITATTN_ERR_NULL_POINTER = -1,     /* a required pointer is NULL */
  VITATTN_ERR_BAD_SIZE = -2,         /* B, H or N negative */
  VITATTN_ERR_UNSUPPORTED_D = -3,    /* D is not 64 or 72 */
  VITATTN_ERR_BAD_SCALE = -4,        /* scale is NaN or infinite */
  VITATTN_ERR_BAD_LAYOUT = -5,       /* unknown layout, or k/v given with the packed layout */
  VITATTN_ERR_MISALIGNED = -6,       /* a pointer is not 16-byte aligned */
  VITATTN_ERR_TOO_LARGE = -7,        /* the problem exceeds the launch limits */
  VITATTN_ERR_LAUNCH = -8,           /* the HIP launch reported an error */
  VITATTN_ERR_OVERLAP = -9,          /* out overlaps an input buffer */
  VITATTN_ERR_GRAPH = -10,           /* recording or launching a HIP graph failed */
  VITATTN_ERR_UNSUPPORTED_SHAPE = -11 /* vitattn_linear: K or Nout not supported */
};

/*
 * vitattn_fwd -- O = softmax(scale * Q K^T) V for all B*H (image, head) pairs.
 *
 *   qkv_or_q  device pointer, bf16 (fp16 with VITATTN_DTYPE_FP16).  Separate
 *             layout: Q [B][H][N][D].
 *             Packed layout: the fused qkv buffer [B][N][3][H][D].
 *   k, v      device pointers, [B][H][N][D] for the separate layout;
 *             must be NULL for the packed layout.
 *   out       device pointer, same format, written in full: [B][H][N][D] (separate)
 *             or [B][N][H][D] (packed).  Must not overlap any input.
 *   B, H, N   images, heads, tokens.  Any N >= 1 (not only tile multiples)
 *             up to 2^24; B*H*N at most 2^40 and B*H*ceil(N/32) at most
 *             2^30 (else VITATTN_ERR_TOO_LARGE).  B, H or N equal to 0 is
 *             an empty problem: returns VITATTN_OK and launches nothing (its
 *             pointers may then be NULL).
 *   D         head dimension: 64 or 72.
 *   scale     logit scale, any finite value (usually 1/sqrt(D)); 0 gives
 *             uniform attention.
 *   layout    VITATTN_LAYOUT_SEPARATE_BHND or VITATTN_LAYOUT_PACKED_BN3HD,
 *             optionally OR-ed with VITATTN_DTYPE_FP16.
 *   stream    a hipStream_t (NULL = the null stream).  The call only
 *             enqueues one kernel on it and returns without waiting.
 *
 * Ownership: the caller owns every buffer and keeps it alive until the
 * enqueued work has finished.  All pointers must be 16-byte aligned.
 *
 * Errors: every argument is checked on the host before anything is
 * launched, and a failed check returns its negative code with no device
 * work.  VITATTN_ERR_LAUNCH means the runtime rejected the launch (for
 * instance, no gfx950 device is current).  Faults inside the kernel are
 * reported, as for any HIP kernel, by the next synchronising HIP call.
 */
int vitattn_fwd(const void* qkv_or_q, const void* k, const void* v, void* out, int B, int H,
                int N, int D, float scale, int layout, void* stream);

/*
 * vitattn_fwd_shape -- describes the launch vitattn_fwd makes for these sizes
 * on the current device, without launching anything: how the (image, head,
 * query) work is cut into work items and workgroups (the kernel's work
 * decomposition follows the memory-aware tiling the Pi0 Flash Attention
 * tutorial, section 1, credits for the speed-up).  For tests and benchmarks
 * that name the kernel path they exercise.
 *
 *   waves       receives the waves of 64 lanes per workgroup: 1, 2 or 4.
 *   split_keys  receives 1 when the waves of a workgroup share one block of
 *               32 queries and split its keys (short sequences), else 0
 *               (each wave then owns 32 queries of the block).
 *   items       receives the number of work items (image, head, query block).
 *   workgroups  receives the number of workgroups launched: one per item, or
 *               fewer, each looping over several items.
 *
 * B, H, N, D and layout as for vitattn_fwd.  Errors: VITATTN_ERR_NULL_POINTER
 * (an output pointer is NULL), and the size, head-dimension, layout and
 * limit codes vitattn_fwd returns for the same sizes; nothing is written
 * then.  With no usable device the count of compute units is unknown and
 * the description is that of a launch with one workgroup per item.
 */
int vitattn_fwd_shape(int B, int H, int N, int D, int layout, int* waves, int* split_keys,
                      int* items, int* workgroups);

/*
 * Plans: a fixed sequence of forward calls recorded once into a HIP graph and
 * launched as one unit.  A vision encoder runs the same attention shape once
 * per layer on buffers that stay in place, so per-call launch work can be
 * paid once: the FluxVLA "Inference acceleration" tutorial (section 2,
 * CUDA Graph capture; section 3, preallocated outputs that stay valid inside
 * a graph) and Realtime-VLA (section 1.2.1) run whole model stages as one
 * captured graph for this reason.
 */
typedef struct vitattn_plan_s* vitattn_plan;

/*
 * vitattn_plan_create -- records `layers` calls of vitattn_fwd, call l with
 * the buffers qkv_or_q[l], k[l], v[l], out[l] and the shared sizes, scale and
 * layout, into one executable HIP graph.  Nothing is computed.
 *
 *   plan      receives the new plan, or NULL on error.
 *   layers    number of recorded calls, >= 1.
 *   qkv_or_q, out
 *             host arrays of `layers` device pointers, as for vitattn_fwd.
 *   k, v      host arrays of `layers` device pointers for the separate
 *             layout; must be NULL (the arrays themselves) for the packed
 *             layout.
 *   B, H, N, D, scale, layout
 *             as for vitattn_fwd, the same for every call.
 *
 * Every call is checked as vitattn_fwd checks it before anything is
 * recorded; the first failing check's code is returned.  Recording uses a
 * private stream of default priority on the current device, which the plan
 * is then bound to.  VITATTN_ERR_GRAPH: the HIP runtime refused to record or
 * instantiate the graph (or host memory ran out).
 *
 * Ownership: the caller owns the plan and every buffer it names; the buffers
 * must stay allocated, at the same addresses, for as long as the plan is
 * launched (their contents may change between launches: each launch reads
 * the inputs as they are then).
 */
int vitattn_plan_create(vitattn_plan* plan, int layers, const void* const* qkv_or_q,
                        const void* const* k, const void* const* v, void* const* out, int B,
                        int H, int N, int D, float scale, int layout);

/*
 * vitattn_plan_launch -- enqueues all recorded calls, in order, on `stream`
 * (a hipStream_t of the plan's device; NULL = the null stream) and returns
 * without waiting.  Output is bitwise what the same vitattn_fwd calls give.
 * Errors: VITATTN_ERR_NULL_POINTER (plan is NULL), VITATTN_ERR_GRAPH (the
 * runtime rejected the graph launch).
 */
int vitattn_plan_launch(vitattn_plan plan, void* stream);

/*
 * vitattn_plan_destroy -- frees the plan (NULL is allowed and ignored).  Work
 * already enqueued by vitattn_plan_launch still completes.
 */
int vitattn_plan_destroy(vitattn_plan plan);

/*
 * vitattn_linear -- the linear layers on either side of the attention in a
 * ViT block, on the same hardware path (bf16 or fp16 MFMA, fp32 accumulate):
 *
 *     out[m][n] = sum_k x[m][k] * w[n][k] + bias[n] + residual[m][n]
 *
 * Two uses: the block's fused qkv projection, whose [M][3*H*D] output with
 * M = B*N is exactly the packed [B][N][3][H][D] buffer vitattn_fwd reads
 * (the FluxVLA "Inference acceleration" tutorial, section 1, fuses this
 * projection; the Pi0 Flash Attention tutorial, section 3.2, feeds the
 * attention from it), and the output projection with its bias and the
 * block's residual add in one pass (the same FluxVLA tutorial, section 3).
 *
 *   x         device pointer, [M][K] row-major (tokens x input features).
 *   w         device pointer, [Nout][K] row-major: the layer's weight as
 *             stored (output features x input features).
 *   bias      device pointer to [Nout], or NULL for no bias.
 *   residual  device pointer to [M][Nout], or NULL for none.  May be equal
 *             to `out` (an in-place residual add) but must not overlap it
 *             otherwise.
 *   out       device pointer, [M][Nout], written in full; must not overlap
 *             x, w or bias.
 *   M, K, Nout  sizes: M >= 0 (any value), K a positive multiple of 32,
 *             Nout a multiple of 8 (else VITATTN_ERR_UNSUPPORTED_SHAPE);
 *             M * K and Nout * K below 2^31 elements.  M or Nout equal to
 *             0 is an empty problem (returns VITATTN_OK, launches nothing).
 *   flags     0 for bf16 tensors, VITATTN_DTYPE_FP16 for fp16 (all tensors
 *             in the one format); other bits: VITATTN_ERR_BAD_LAYOUT.
 *   stream    a hipStream_t (NULL = the null stream); the call enqueues one
 *             kernel and returns without waiting.
 *
 * Numerics: 16-bit inputs, fp32 accumulation of the products, bias and
 * residual added in fp32, one rounding (nearest even) to the output format.
 * Deterministic.  Ownership, alignment (16 bytes) and error behaviour as
 * for vitattn_fwd.
 */
int vitattn_linear(const void* x, const void* w, const void* bias, const void* residual,
                   void* out, int M, int K, int Nout, int flags, void* stream);

/* A fixed English sentence for a status code ("unknown status" for any
 * other value); static storage, never freed.  For the messages a caller
 * shows when a call fails (Pi0 Flash Attention tutorial, section 5.2: each
 * failure has a readable cause). */
const char* vitattn_strerror(int status);

/* Library version as 10000*major + 100*minor + patch, so that a caller can
 * check which build it loaded (the same section 5.2 table traces an import
 * failure to a library version mismatch). */
int vitattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VITATTN_H */
