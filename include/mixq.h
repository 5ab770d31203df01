/*
 * mixq.h -- C ABI of the MI355X (gfx950) mixed-precision linear layer
 *
 *     Y = X . W^T      X: fp16 [M, K] activations, W: fp16 [N, K] weights
 *
 * computed the MixQ way: activations quantized per token to INT8 from an
 * amax pass; the few input channels holding outliers (|x| above a threshold)
 * split out, in channel order, into a small FP16 matrix; the bulk multiplied
 * as INT8 x INT8 (or INT8 x INT4 weights) with INT32 accumulation, the
 * outlier columns as FP16 x FP16; the low-precision result dequantized,
 * scaled and added to the outlier product in one fused epilogue.  The outlier
 * channel set is cached across calls and re-detected only when the amax of
 * the uncached channels exceeds the threshold.
 *
 * Sources (cited by page title and section; they print no API, so the calls
 * below are this library's own):
 *   MixQ article -- news article on MixQ, "一键部署LLM混合精度推理，端到端吞吐比
 *     AWQ最大提升6倍！": section "研究背景：已有量化技术总结", Fig. 5 (split of
 *     the product into a low-bit part and an FP16 outlier part, summed);
 *     section "MixQ的解决方案": Fig. 9 (outliers recur in fixed channels across
 *     decode steps), the amax-versus-threshold paragraph (the amax that
 *     quantization computes anyway tells whether outliers exist), Fig. 10
 *     (equivalent graph transform that skips detection), Fig. 11 (outliers
 *     concatenated, order preserved, into a new matrix), Fig. 12 (dequantize,
 *     scale and add fused in registers).
 *   FP6 explainer -- "DeepSpeed FP6以 FP6 量化与 TC-FPx 全栈 GPU Kernel 为核心的
 *     LLM 推理服务加速": section 2.3 (unsupported shapes rejected with an
 *     explicit error), section 3 (explicit error on unsupported hardware;
 *     per-output-channel scale = max|w| over the code range, zero scale -> 1).
 *   QServe notes -- reading notes on QServe W4A8KV4: sections
 *     "寄存器压力和并行性" and "小结" (INT4 weights decoded to INT8 inside the
 *     GEMM main loop so that every product runs on INT8 matrix units).
 *
 * Conventions for every call
 *   - Device pointers point to memory of the current HIP device; structs are
 *     host memory passed by pointer and read during the call only.
 *   - The library never allocates, frees or synchronizes.  Every buffer is
 *     owned by the caller.  Work is enqueued on `stream` (a hipStream_t; NULL
 *     = the default stream) and runs asynchronously.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns an error and enqueues nothing.
 *   - Calls on different streams are safe when they touch disjoint buffers.
 *     Two calls that share an activation state or a packed weight must be
 *     ordered (same stream, or events).
 *   - Return value: MIXQ_OK or one of the MIXQ_ERR_* codes below.  Nothing is
 *     printed and no exception or abort crosses the ABI.
 */
#ifndef MIXQ_H
#define MIXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
enum {
    MIXQ_OK = 0,
    MIXQ_ERR_INVALID_ARG = 1,        /* null pointer, size <= 0, bad enum, ...   */
    MIXQ_ERR_UNSUPPORTED_SHAPE = 2,  /* K not a multiple of 64, or a size whose
                                        byte offsets would leave 32 bits        */
    MIXQ_ERR_UNSUPPORTED_DEVICE = 3, /* current device is not gfx950            */
    MIXQ_ERR_NO_DEVICE = 4,          /* no HIP device visible                    */
    MIXQ_ERR_HIP = 5,                /* a HIP launch reported an error          */
    MIXQ_ERR_WORKSPACE = 6           /* a workspace was given but is too small   */
};

/* ---- limits --------------------------------------------------------------- */
#define MIXQ_K_MULTIPLE 64           /* K must be a multiple of this            */
#define MIXQ_K_MAX 65536             /* largest supported K                     */
#define MIXQ_OUTLIER_ALIGN 32        /* outlier matrices padded to this many k  */
#define MIXQ_NORM_K_MAX 32768        /* largest K of mixq_rmsnorm_quantize_act  */

/* flag bits written by mixq_quantize_act into *state->flag */
#define MIXQ_FLAG_FIRED 1            /* gate fired, set grew                    */
#define MIXQ_FLAG_OVERFLOW 2         /* gate fired, but |set| would exceed k_cap;
                                        set left unchanged                      */

#define MIXQ_PROGRESSIVE_GROUP 128   /* channels per group of progressive INT4  */

/* output modes of mixq_gemm_ex */
#define MIXQ_OUT_F32 0               /* Y fp32 [M, N]                            */
#define MIXQ_OUT_SWIGLU_F16 1        /* gated weight: Y fp16 [M, N/2] =
                                        silu(gate) * up                          */
#define MIXQ_OUT_F16 2               /* Y fp16 [M, N]: the fp32 output rounded to
                                        nearest, ties to even                    */
#define MIXQ_OUT_BF16 3              /* Y bf16 [M, N]: likewise                   */

/* mixq_pack_weight modes */
#define MIXQ_PACK_FULL 0             /* quantize all of W and gather outliers   */
#define MIXQ_PACK_OUTLIER_COLS 1     /* only re-gather the outlier columns, and
                                        only if the state's set has changed     */

/*
 * Cached outlier-channel set of one activation stream (MixQ article,
 * "MixQ的解决方案", Fig. 9 and the amax paragraph).  All pointers are device
 * memory, owned by the caller and zero-filled once before the first call
 * (an empty set); after that only the library writes them.  The set only
 * grows: channels found by a firing gate are added to it.
 */
typedef struct mixq_act_state {
    int32_t *idx;      /* [k_cap]  outlier channel ids, ascending; first *count valid */
    int32_t *count;    /* [1]      size of the set                                   */
    int32_t *flag;     /* [1]      MIXQ_FLAG_* bits of the last quantize call        */
    uint32_t *bitmap;  /* [mixq_bitmap_words(K)]  bit k%32 of word k/32 = channel k  */
    uint32_t *work;    /* [mixq_state_work_words(K)]  library scratch: detection
                          bits, rank prefix of the bitmap, counters, and the
                          serial of the committed set (unique per commit within
                          the process, 0 for the empty set of a zeroed state)  */
    int32_t k_cap;     /* host value: capacity of the set, 0 <= k_cap <= K           */
} mixq_act_state;

/* Number of per-block version slots of a packed weight (see mixq_weight.k_out). */
#define MIXQ_GATHER_SLOTS 256

/*
 * A packed weight (FP6 explainer, section 3: weights quantized once, per
 * output channel, symmetric; MixQ article, Fig. 11: FP16 columns of the
 * outlier channels kept beside them, in channel order).  Device buffers are
 * owned by the caller; mixq_pack_weight fills them.
 */
typedef struct mixq_weight {
    void *wq;          /* bits 8: int8 [N, K] row-major codes in [-127, 127];
                          bits 4: K-tile-major inside 32-row blocks, uint8
                          [ceil(N/32)][K/64][32 rows][32 bytes]: row n's 64 k of
                          tile k/64 are the 32 bytes at block n/32, row n%32, as
                          8 words in k order; each word holds 8 consecutive k:
                          byte j = (q[k+j] & 15) | (q[k+j+4] & 15) << 4, codes
                          in [-7, 7]; rows of the last block past N unused    */
    float *s_w;        /* [N] per-output-channel scale                            */
    uint16_t *w_out;   /* fp16 [N, mixq_outlier_ld(k_cap)]: W at the outlier
                          channels in set order, then zeros                       */
    int32_t *k_out;    /* [MIXQ_GATHER_SLOTS] serial of the state set each slice
                          of w_out was gathered for; zero-fill once               */
    int32_t bits;      /* 8 or 4                                                  */
    int64_t N, K;
    int32_t k_cap;     /* must equal the k_cap of the states it is used with      */
    int32_t gated;     /* 0: rows of W in order.  1: W = [W_gate; W_up] ([2I, K],
                          I = N/2, N a multiple of 64), packed with 32-row blocks
                          of gate and up rows interleaved (packed row p holds W
                          row 32*(p/64) + p%64 for p%64 < 32, else
                          I + 32*(p/64) + p%64 - 32); wq, s_w and w_out all
                          follow the packed order.  Needed by
                          MIXQ_OUT_SWIGLU_F16.                                    */
    int32_t group;     /* 0: INT4 codes are symmetric per channel (as above).
                          MIXQ_PROGRESSIVE_GROUP (bits 4 only): progressive
                          group-wise INT4 (QServe page, progressive group
                          quantization): per channel to INT8 with the range
                          [-119, 119] (s_w = max|W[n,:]| / 119), then per group
                          of 128 channels a 4-bit value u in [0, 15], an integer
                          scale s2 in [1, 16] and zero z in [0, 15]; the product
                          uses the INT8 code (u - z) * s2.  wq holds u in the
                          INT4 nibble layout.                                      */
    uint16_t *gsz;     /* group != 0: [K/128, N] (group-major), s2 | z << 8 for
                          each group and row (device memory, written by
                          mixq_pack_weight); N * K/128 * 2 bytes < 2^31        */
    const int32_t *rmap; /* NULL, or a row subset: [N] device array, the W row
                          each packed row quantizes, which is also the Y column
                          the product writes for it.  Output-feature mixed
                          precision (MixLLM page) is two such weights over one
                          W: the salient rows at bits 8 and the others at bits
                          4, each multiplied by its own mixq_gemm call into the
                          same Y.  An entry outside [0, n_out) packs zeros and
                          writes nothing.  Bits 8, or bits 4 with a group; not
                          with gated weights or the SwiGLU output.             */
    int32_t n_out;     /* rmap != NULL: rows of W = output features (columns of
                          Y); ldy >= n_out                                        */
} mixq_weight;

/* ---- size helpers (pure host functions) ---------------------------------- */
/* Row length of X_out and w_out: k_cap rounded up to MIXQ_OUTLIER_ALIGN. */
int64_t mixq_outlier_ld(int32_t k_cap);
/* Number of 32-bit words of a state's bitmap: ceil(K / 32). */
int64_t mixq_bitmap_words(int64_t K);
/* Number of 32-bit words of a state's work area: 2 * ceil(K / 32) + 4. */
int64_t mixq_state_work_words(int64_t K);
/* Bytes of mixq_weight.wq: N*K for 8 bits, ceil(N/32)*32*K/2 for 4 bits
 * (whole 32-row blocks); 0 if invalid. */
size_t mixq_packed_weight_bytes(int64_t N, int64_t K, int32_t bits);

/*
 * mixq_quantize_act -- amax, gate, detection and per-token INT8 quantization
 * with the outlier split (MixQ article, "MixQ的解决方案": the amax paragraph
 * and Figs. 10-11; Fig. 5 for the split).
 *
 * For each token m:  a_m = max |X[m,k]| over channels k not in the set;
 * s_x[m] = a_m / 127 and r = 127 / a_m (both single IEEE fp32 divisions; a_m = 0
 * gives s_x = r = 1); Xq[m,k] = 0 for k in the set, else
 * clamp(round_half_even(X[m,k] * r), -127, 127);  X_out[m, j] = X[m, idx[j]]
 * for j < count, zeros up to the next multiple of MIXQ_OUTLIER_ALIGN.
 * Before quantizing, the gate compares the amax of the uncached channels with
 * `threshold` (strictly greater fires).  If it fires, every channel with some
 * |X[m,k]| > threshold joins the set (if the set would exceed k_cap, it is
 * left unchanged and MIXQ_FLAG_OVERFLOW is raised) and the call quantizes
 * with the new set.  *state->flag is rewritten by every call.
 *
 *   X        fp16 [M, ldx] device, row-major, read-only; finite values
 *   M        tokens, >= 1;   K: channels, multiple of 64, <= MIXQ_K_MAX
 *   ldx      row stride of X in elements, >= K
 *   threshold finite, >= 0
 *   state    the cached set (see mixq_act_state); k_cap <= K
 *   Xq       int8 [M, K] device, written
 *   s_x      fp32 [M] device, written
 *   X_out    fp16 [M, mixq_outlier_ld(k_cap)] device, written up to the padded
 *            set size; may be NULL when k_cap == 0
 * Errors: MIXQ_ERR_INVALID_ARG, MIXQ_ERR_UNSUPPORTED_SHAPE, MIXQ_ERR_NO_DEVICE,
 *         MIXQ_ERR_UNSUPPORTED_DEVICE, MIXQ_ERR_HIP.
 */
int mixq_quantize_act(const uint16_t *X, int64_t M, int64_t K, int64_t ldx, float threshold,
                      const mixq_act_state *state, int8_t *Xq, float *s_x, uint16_t *X_out,
                      void *stream);

/*
 * mixq_quantize_act_regather -- mixq_quantize_act followed by
 * mixq_pack_weight(W, w->N, K, w->bits, state, MIXQ_PACK_OUTLIER_COLS, w),
 * in two kernel launches instead of three: the launch that re-quantizes
 * after a firing gate also re-gathers the weight's outlier columns (MixQ
 * article, Fig. 11), and on a call whose set stands it checks them (no-op
 * unless they hold another set).  Results are those of the two calls.
 *
 *   X, M, K, ldx, threshold, state, Xq, s_x, X_out   as mixq_quantize_act
 *   W, w      as mixq_pack_weight (w->K == K, w->k_cap == state->k_cap)
 * Errors: as mixq_quantize_act and mixq_pack_weight.
 */
int mixq_quantize_act_regather(const uint16_t *X, int64_t M, int64_t K, int64_t ldx,
                               float threshold, const mixq_act_state *state, int8_t *Xq,
                               float *s_x, uint16_t *X_out, const uint16_t *W,
                               const mixq_weight *w, void *stream);

/*
 * mixq_rmsnorm_quantize_act -- mixq_quantize_act applied to the RMS-normalised
 * tokens, in the same pass over memory: the amax that the quantization needs
 * is fused into the operation before the layer (MixQ article, "MixQ的解决方案",
 * the paragraph after the amax test).  For a LLaMA linear that operation is
 * RMSNorm; the normalised X is never written to memory.
 *
 * For each token m, with every rounding fixed so that the result is unique:
 *   S = sum_k H[m,k]^2 exactly, rounded once to binary64;
 *   ms = fp32(S / K);  rstd[m] = 1 / sqrt(ms + eps) in binary32 (0 when
 *   ms + eps == 0, i.e. an all-zero token with eps = 0);
 *   X[m,k] = fp16(fp16(H[m,k] * rstd[m]) * gamma[k])  (binary32 product
 *   rounded to fp16, then the fp16 product rounded to fp16);
 * then everything mixq_quantize_act does, on X: gate, detection, Xq, s_x and
 * X_out (which holds normalised values).
 *
 *   H        fp16 [M, ldh] device, row-major, read-only; finite, and every
 *            normalised value must be finite in fp16
 *   M, K     as mixq_quantize_act, and K <= MIXQ_NORM_K_MAX
 *   ldh      row stride of H in elements, >= K
 *   gamma    fp16 [K] device, 16-byte aligned, read-only
 *   eps      finite, >= 0
 *   threshold, state, Xq, s_x, X_out   as mixq_quantize_act
 *   rstd     fp32 [M] device, written
 * Errors: as mixq_quantize_act; MIXQ_ERR_INVALID_ARG also for a null gamma or
 *         rstd or a bad eps; MIXQ_ERR_UNSUPPORTED_SHAPE also for K above
 *         MIXQ_NORM_K_MAX or a misaligned gamma.
 */
int mixq_rmsnorm_quantize_act(const uint16_t *H, int64_t M, int64_t K, int64_t ldh,
                              const uint16_t *gamma, float eps, float threshold,
                              const mixq_act_state *state, int8_t *Xq, float *s_x,
                              uint16_t *X_out, float *rstd, void *stream);

/*
 * mixq_add_rmsnorm_quantize_act -- the residual update of a LLaMA block
 * followed by mixq_rmsnorm_quantize_act, in one pass over memory: the whole
 * operation before the layer, into which the MixQ article ("MixQ的解决方案",
 * the paragraph after the amax test) lets the amax be fused.
 *
 *   H[m,k] = fp16(R[m,k] + D[m,k])   (the exact sum rounded once, ties to
 *                                     even), written out as the new residual;
 *   then everything mixq_rmsnorm_quantize_act does, on H.
 *
 *   R, D     fp16 [M, ldr] and [M, ldd] device, row-major, read-only; finite
 *            sums
 *   H        fp16 [M, ldh] device, written; it must not overlap R or D (a
 *            ping-pong pair of residual buffers replaces an in-place update)
 *   ldr, ldd, ldh  row strides in elements, >= K, multiples of 8; R, D, H
 *            16-byte aligned
 *   M, K, gamma, eps, threshold, state, Xq, s_x, X_out, rstd
 *            as mixq_rmsnorm_quantize_act
 * Errors: as mixq_rmsnorm_quantize_act; MIXQ_ERR_INVALID_ARG also for a null
 *         D or H, a stride below K, or H overlapping R or D;
 *         MIXQ_ERR_UNSUPPORTED_SHAPE also for misaligned D or H or strides.
 */
int mixq_add_rmsnorm_quantize_act(const uint16_t *R, int64_t ldr, const uint16_t *D, int64_t ldd,
                                  uint16_t *H, int64_t ldh, int64_t M, int64_t K,
                                  const uint16_t *gamma, float eps, float threshold,
                                  const mixq_act_state *state, int8_t *Xq, float *s_x,
                                  uint16_t *X_out, float *rstd, void *stream);

/*
 * mixq_pack_weight -- per-output-channel symmetric quantization of W and the
 * FP16 outlier columns (FP6 explainer, section 3; MixQ article, Fig. 11).
 *
 *   s_w[n] = alpha_n / Q and rho = Q / alpha_n, alpha_n = max_k |W[n,k]| over
 *   all K, Q = 127 (bits 8) or 7 (bits 4), alpha_n = 0 gives 1;
 *   code = clamp(round_half_even(W[n,k] * rho), -Q, Q), stored as documented
 *   in mixq_weight;  w_out[n, j] = W[n, idx[j]] for j < count, then zeros.
 *
 *   W      fp16 [N, K] device, row-major (ld = K); [w->n_out, K] when w->rmap
 *          is set (packed row n then quantizes W row rmap[n]).  Keep it: the
 *          outlier columns are gathered from it again when the set grows.
 *   N, K   >= 1; K multiple of 64, <= MIXQ_K_MAX; N = w->N (the packed row
 *          count: the length of rmap when it is set)
 *   bits   8 or 4
 *   state  the activation state whose set selects the outlier columns
 *   mode   MIXQ_PACK_FULL: everything.  MIXQ_PACK_OUTLIER_COLS: re-gather
 *          w_out only, decided on the device (no host sync): it runs when
 *          the serial of the state's committed set differs from the one the
 *          columns were gathered for, and is a no-op otherwise -- a set that
 *          grew, a reset state, or another state whose set has the same size
 *          all count as changed.  Call it after each mixq_quantize_act and
 *          before mixq_gemm.
 *   w      the packed weight; w->N, w->K, w->bits, w->k_cap must match;
 *          w->gated selects the row order (see mixq_weight) and must be the
 *          same in the FULL call and every OUTLIER_COLS call
 * Errors: as mixq_quantize_act; MIXQ_ERR_INVALID_ARG also for w->gated not 0
 *         or 1, w->group not 0 or MIXQ_PROGRESSIVE_GROUP, a group with bits 8,
 *         or a null w->gsz with a group, and for a w->rmap with a gated
 *         weight, with symmetric INT4 or with n_out < 1;
 *         MIXQ_ERR_UNSUPPORTED_SHAPE for a gated N
 *         not a multiple of 64 or a group not dividing K.
 */
int mixq_pack_weight(const uint16_t *W, int64_t N, int64_t K, int32_t bits,
                     const mixq_act_state *state, int32_t mode, const mixq_weight *w,
                     void *stream);

/*
 * mixq_gemm -- the two products and the fused epilogue (MixQ article, Fig. 5
 * and Fig. 12):
 *
 *   acc[m,n] = sum_k Xq[m,k] * Wq[n,k]                 (exact, int32)
 *   Y[m,n]   = float(acc) * s_x[m] * s_w[n] + sum_{j < count} X_out[m,j] * w_out[n,j]
 *
 * with INT8 x INT8 (INT4 weights decoded to INT8 in the kernel) matrix-core
 * products accumulated in int32, the outlier product on FP16 matrix cores
 * accumulated in fp32, and the dequantize/scale/add done in registers.  The
 * set size is read on the device from state->count (no host sync).
 *
 *   Xq, s_x, X_out  as written by mixq_quantize_act for the same state
 *   state           the activation state (count and k_cap are used)
 *   w               packed weight, gathered for the current set
 *   M               tokens, >= 1
 *   Y               fp32 [M, ldy] device; ldy >= N.  With w->rmap: ldy >=
 *                   w->n_out, and only the columns rmap names are written
 *   acc_debug       NULL, or int32 [M, N] device: also receives acc, in
 *                   packed row order
 * Errors: as mixq_quantize_act; MIXQ_ERR_INVALID_ARG also for a w->rmap
 *         that mixq_pack_weight would reject; MIXQ_ERR_UNSUPPORTED_SHAPE also
 *         when 256 rows of Y span 2^31 bytes or more (ldy * 4 * 256 for fp32
 *         output, ldy * 2 * 256 for 16-bit output: the kernel's store offsets
 *         within a tile are 32-bit), or when the launch would need more than
 *         2^31 - 1 blocks.
 */
int mixq_gemm(const int8_t *Xq, const float *s_x, const uint16_t *X_out,
              const mixq_act_state *state, const mixq_weight *w, int64_t M, float *Y,
              int64_t ldy, int32_t *acc_debug, void *stream);

/*
 * mixq_gemm_ws -- mixq_gemm with a split-K workspace, for thin products (few
 * tokens: the decode phase).  FP6 explainer, sections 2.2-2.3: such GEMMs
 * leave most compute units idle unless K is split, the partial results being
 * reduced through a workspace.
 *
 * When the product (INT8 weights, K a multiple of 256) has fewer 128 x 128
 * output tiles than the device has compute units, each tile's K range is
 * split in two blocks.  Both store their exact int32 partial tile in ws; the
 * second to finish adds the other's and runs the epilogue.  No block waits
 * for another.  Integer partial sums make acc and Y bit-identical to the
 * unsplit product.
 *
 * A large product whose 256 x 256 tiles need one round of the device plus a
 * short second one runs the columns that fill one round on 256 x 256 tiles
 * and the remaining columns as a second launch of 128 x 128 tiles (with or
 * without ws); with ws, that launch also splits K two or four ways in the
 * same way, so that its blocks fill the device.
 *
 * Otherwise, or when ws is NULL, the call is mixq_gemm.
 *
 *   ws        NULL, or device memory of ws_bytes, 16-byte aligned; its first
 *             4096 bytes (tile counters) must be zero-filled once by the
 *             caller, after which every completed call leaves them zero.
 *             Calls sharing a ws must not overlap (one stream, or serialized).
 *   ws_bytes  at least mixq_gemm_workspace_bytes(M, N, K, bits) (N = w->N)
 * Other arguments: as mixq_gemm.
 * Errors: as mixq_gemm; MIXQ_ERR_WORKSPACE when ws is given and the product
 *         splits but ws_bytes is below what the split needs (nothing is
 *         enqueued).
 */
int mixq_gemm_ws(const int8_t *Xq, const float *s_x, const uint16_t *X_out,
                 const mixq_act_state *state, const mixq_weight *w, int64_t M, float *Y,
                 int64_t ldy, int32_t *acc_debug, void *ws, size_t ws_bytes, void *stream);

/*
 * mixq_gemm_ex -- mixq_gemm_ws with a choice of output.  MIXQ_OUT_F32 is
 * mixq_gemm_ws.  MIXQ_OUT_F16 and MIXQ_OUT_BF16 write the same layer output
 * as 16-bit values, each the fp32 result rounded to nearest with ties to
 * even (the pages' systems hand 16-bit activations to the next layer; the
 * FP6 explainer, section 3, runs its linear layers into pre-allocated fp16
 * outputs).  MIXQ_OUT_SWIGLU_F16 is for the fused gate-and-up
 * projection of a LLaMA MLP (the gated linear layer the FP6 explainer's
 * section 3 runs as one double-output kernel): w must be packed gated, and
 * the epilogue writes, for each token m and output j < N/2,
 *   Y[m, j] = fp16( silu(g) * u ),  silu(g) = g / (1 + e^-g),
 * where g and u are the layer outputs (dequantized integer product plus
 * outlier product, in fp32) of gate row j and up row j -- the same values
 * MIXQ_OUT_F32 writes, taken in pairs in the epilogue.  silu is evaluated in
 * fp32 with the hardware exponential and reciprocal, whose error is far
 * below the fp16 rounding that follows.  The fp32 gate and up outputs never
 * reach memory.
 *
 *   Y         MIXQ_OUT_F32: fp32 [M, ldy], ldy >= N.
 *             MIXQ_OUT_F16 / MIXQ_OUT_BF16: fp16 / bf16 [M, ldy], ldy >= N.
 *             MIXQ_OUT_SWIGLU_F16: fp16 [M, ldy], ldy >= N/2.
 *   out_mode  one of the four MIXQ_OUT_* modes
 *   acc_debug as mixq_gemm, in the packed (interleaved) column order
 * Other arguments: as mixq_gemm_ws (ws may be NULL).
 * Errors: as mixq_gemm_ws; MIXQ_ERR_INVALID_ARG also for an unknown
 *         out_mode, MIXQ_OUT_SWIGLU_F16 with a weight not packed gated, any
 *         16-bit output with a row subset, or ldy below the output's columns.
 */
int mixq_gemm_ex(const int8_t *Xq, const float *s_x, const uint16_t *X_out,
                 const mixq_act_state *state, const mixq_weight *w, int64_t M, void *Y,
                 int64_t ldy, int32_t out_mode, int32_t *acc_debug, void *ws, size_t ws_bytes,
                 void *stream);

/*
 * mixq_gemm_noalloc -- mixq_gemm_ex with no workspace argument and no
 * allocation of any kind, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The split-K workspace that mixq_gemm_ex takes from the caller
 * is a file-scope device array of the library instead, of
 * mixq_gemm_scratch_bytes() bytes: 4096 bytes of tile counters and 512
 * partial tiles of 64 KiB (32 MiB + 4 KiB), which covers every split the
 * library plans on a 256-CU MI355X (at most two partials per compute unit).
 * Every GPU the library runs on holds its own copy until the process ends.
 * The first call on a device takes the array's address
 * (hipGetSymbolAddress) and clears its counters with a fill kernel on
 * `stream`; later calls launch only the GEMM.  Calls on one device share
 * the array: two of them that overlap in time (different streams without
 * ordering) race and give wrong results -- order them.
 *
 *   Arguments: as mixq_gemm_ex without ws / ws_bytes.
 * Errors: as mixq_gemm_ex; MIXQ_ERR_WORKSPACE if a product's split needed
 *         more than the array holds (not reachable on a 256-CU device);
 *         MIXQ_ERR_HIP if the array's address cannot be taken.
 */
int mixq_gemm_noalloc(const int8_t *Xq, const float *s_x, const uint16_t *X_out,
                      const mixq_act_state *state, const mixq_weight *w, int64_t M, void *Y,
                      int64_t ldy, int32_t out_mode, int32_t *acc_debug, void *stream);

/* Bytes of the device array mixq_gemm_noalloc uses in place of ws. */
size_t mixq_gemm_scratch_bytes(void);

/* Workspace bytes mixq_gemm_ws needs to split this product on a device with
 * 256 compute units (MI355X): 4096 bytes of tile counters plus, per split
 * 128 x 128 output tile, one 64 KiB partial tile per part (two for a thin
 * product, two or four for the tail of a large one); 0 when nothing is
 * split. */
size_t mixq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t bits);

/*
 * mixq_set_gemm_variant -- testing hook.  Every later GEMM call in the
 * process uses kernel variant `variant` (1..6) instead of the automatic
 * choice (0, the default and the only mode meant for use): 1 = 256 x 256
 * tiles with 64-byte K steps, 2 = 128 x 128 tiles with 64-byte K steps,
 * 3 = 256 x 256 software-pipelined (INT4 weights), 4 = 256 x 256 with
 * 128-byte K pairs (INT8 weights), 5 = 128 x 128 with 128-byte K pairs (INT8;
 * K split under mixq_gemm_ws), 6 = 128 x 128 software-pipelined (INT4).  A
 * variant whose loader does not fit the call (K not a multiple of 128, or
 * the other weight width) falls back to one that does.  All variants give
 * bit-identical accumulators; the hook lets tests cover each of them on
 * small shapes.  Not thread-safe with respect to GEMM calls in flight on
 * other host threads.
 * Errors: MIXQ_ERR_INVALID_ARG for an id outside 0..6.
 */
int mixq_set_gemm_variant(int32_t variant);

/*
 * mixq_set_clock_record -- measurement hook.  While buf is set, every later
 * GEMM launch in the process has its blocks b < n_blocks write four int64
 * stamps to buf[4b .. 4b+3]: the shader-clock counter (s_memtime) at the
 * block's entry and exit, then the 100 MHz real-time counter
 * (s_memrealtime) at entry and exit, so that the engine clock of the
 * product itself is (clock delta) / (real-time delta / 100 MHz).  Each
 * launch overwrites the records of the last.  buf: device memory of
 * 4 * n_blocks int64; (NULL, 0) turns the hook off (the default).
 * Errors: MIXQ_ERR_INVALID_ARG for a null buf with n_blocks > 0 or the
 *         reverse, or n_blocks < 0.
 */
int mixq_set_clock_record(int64_t *buf, int32_t n_blocks);

/*
 * mixq_mfma_probe -- measurement aid: the GEMM main loop's INT8 matrix-core
 * stream with no memory traffic.  The MixQ article (section "MixQ的解决方案",
 * Fig. 14) states its kernels' throughput against the hardware's peak; the
 * published MI355X peak assumes the 2.4 GHz engine clock, which the board
 * lowers under sustained matrix work by an amount that depends on the
 * operand bits.  This call measures the matrix-core rate at the clock the
 * board sustains, on given operand bytes (for instance a workload's own Xq
 * and packed weight), as a ceiling the GEMM's memory traffic does not enter.
 *
 * Each of the blocks x 4 waves (one per SIMD) loads, per lane, eight
 * 16-byte A operands and eight B operands once: operand q (q = 4 ks + i,
 * ks in 0..1, i in 0..3) of wave g (g = 4 block + wave) is bytes
 *   [((8 g + q) * 1024 + 16 lane) mod size, +16)
 * of a (a_bytes) and of b (b_bytes).  It then runs `iters` rounds of 32
 * v_mfma_i32_32x32x32_i8: for ks, for i, for j (0..3):
 *   acc[i][j] += A(ks, i) B(ks, j)^T,
 * where A(ks, i) is the 32 x 32 int8 matrix whose row r holds the operand
 * bytes of lane r (k 0..15) then lane r + 32 (k 16..31), B(ks, j) likewise.
 * acc[i][j] is a 32 x 32 int32 matrix; lane l holds column l % 32 and rows
 * 8 (e / 4) + 4 (l / 32) + e % 4, e in 0..15.  out[256 b + t] receives,
 * for thread t of block b, the sum of that lane's 256 accumulator values,
 * in 32-bit wrapping arithmetic.
 *
 *   a, b      device memory, 16-byte aligned, of a_bytes / b_bytes bytes
 *             (multiples of 16, at least 16)
 *   iters     rounds (>= 1): 32 * iters MFMAs per wave; 128 rounds is the
 *             MFMA count of one wave of the 256 x 256 GEMM at K = 8192
 *   blocks    >= 1; one per compute unit (256 on MI355X) matches the GEMM
 *   out       device int32 [256 * blocks]
 *   clk       NULL, or device int64 [4 * blocks]: per block the shader-clock
 *             counter (s_memtime) before and after the MFMA rounds, then the
 *             100 MHz real-time counter (s_memrealtime) before and after
 *   stream    hipStream_t (NULL = default stream)
 * Errors: MIXQ_ERR_INVALID_ARG for null pointers, iters or blocks < 1, sizes
 *         below 16 or not multiples of 16, or unaligned operands;
 *         MIXQ_ERR_NO_DEVICE / MIXQ_ERR_UNSUPPORTED_DEVICE; MIXQ_ERR_HIP if
 *         the launch fails.
 */
int mixq_mfma_probe(const int8_t *a, int64_t a_bytes, const int8_t *b, int64_t b_bytes,
                    int32_t iters, int32_t blocks, int32_t *out, int64_t *clk, void *stream);

/* Text of a status code (static storage). */
const char *mixq_status_string(int status);

/* MIXQ_OK when the current HIP device is gfx950, else MIXQ_ERR_NO_DEVICE or
 * MIXQ_ERR_UNSUPPORTED_DEVICE (FP6 explainer, section 3: explicit error on
 * unsupported hardware). */
int mixq_check_device(void);

/* ABI version: 100 * major + minor. */
int mixq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MIXQ_H */
