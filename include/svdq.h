/*
 * svdq.h - C ABI of libsvdq: the SVDQuant W4A4 linear layer with its 16-bit
 * low-rank branch fused into the 4-bit branch, for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (SVDQuant paper walkthrough, devpress.csdn.net, eq. (5)):
 *
 *     Y = X W ~= (X diag(lambda)^-1) L1 L2  +  Q(X diag(lambda)^-1) Q(R)  + b
 *
 * with W (K x N) smoothed to W_hat = diag(lambda) W, split by a top-r SVD into
 * L1 L2 (K x r, r x N, kept in bf16) and a residual R = W_hat - L1 L2 that is
 * quantized to 4 bits.  Fused execution (the Nunchaku design, walkthrough
 * Fig. 6): one kernel reads X once to produce the 4-bit activation codes and
 * the down-projection X_hat L1; a second kernel runs the 4-bit GEMM and adds
 * the up-projection (X_hat L1) L2 into the same accumulators.
 *
 * Conventions shared by every call
 *  - Every entry point returns an svdq_status; 0 (SVDQ_OK) is success.  No
 *    C++ exception, abort or exit crosses this boundary.
 *  - Arguments are validated on the host before any GPU work; an invalid call
 *    launches nothing and writes nothing.
 *  - Pointers named d_* are device pointers (HIP device memory of the current
 *    device); all other pointers are host pointers.  The caller owns every
 *    buffer; the library keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Hot
 *    path calls (svdq_act_absmax, svdq_quantize_act, svdq_linear,
 *    svdq_linear_unfused) are asynchronous and stream-ordered: they enqueue
 *    kernels and return.  They allocate nothing and may run concurrently on
 *    different streams when their output buffers differ.
 *  - Tensors are dense row-major with the leading dimension equal to the row
 *    length, and 16-byte aligned.  bf16 is passed as raw 16-bit patterns.
 *  - W is in the paper's orientation, K x N with Y = X W (walkthrough, eq.
 *    (3): X in R^{b x m}, W in R^{m x n}); an nn.Linear weight is its
 *    transpose.
 *  - The device must be gfx950; any other device gives
 *    SVDQ_ERR_UNSUPPORTED_DEVICE (unsupported GPU generations are refused
 *    at load time, as the Diffusers/Nunchaku integration page describes for
 *    its 4-bit operators).
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad enum, alpha out of [0,1] ... */
  SVDQ_ERR_UNSUPPORTED_SHAPE = 2,  /* K, N, r or M outside the supported set */
  SVDQ_ERR_UNSUPPORTED_DEVICE = 3, /* no device, or not gfx950 */
  SVDQ_ERR_BUFFER_TOO_SMALL = 4,   /* prepared / workspace buffer smaller than required */
  SVDQ_ERR_HIP = 5,                /* a HIP runtime call or a launch failed */
  SVDQ_ERR_BAD_BLOB = 6,           /* prepared blob header does not match the descriptor */
  SVDQ_ERR_MISALIGNED = 7          /* a pointer is not 16-byte aligned */
} svdq_status;

/* 4-bit formats (quantizer of eq. (1) of the walkthrough, applied per group
 * along K).
 *  SVDQ_INT4_G64_FP16: signed integer codes in [-7, 7] (q_max = 2^3 - 1),
 *    one fp16 scale per 64 consecutive K elements (the quantization handbook's
 *    "one scale per 64 elements"), s = fp16(max|v| / 7), codes
 *    clamp(round_half_even(v / s)) of the exact quotient; s = 0 -> codes 0.
 *    Eight codes per 32-bit little-endian word (codes k .. k + 7, k % 8 ==
 *    0): code j of the word is the byte c = (q < 0) << 7 | |q| (the FP8
 *    E4M3 bits of q * 2^-9; zero is +0, c = 0); codes 0-3 occupy bits 7 and
 *    0-2 of bytes 0-3, codes 4-7 the same positions rotated left by 4 bits:
 *        word = C0123 | rotl32(C4567, 4)
 *    so word & 0x87878787 and rotr32(word, 4) & 0x87878787 are the E4M3
 *    bytes of codes 0-3 and 4-7.  The words sit where the block order below
 *    puts the bytes of codes k .. k + 7.
 *  SVDQ_FP4_E2M1_G32_E8M0: 4-bit float codes (sign, 2 exponent bits, 1
 *    mantissa bit; q_max = 6 as the walkthrough states for 4-bit floats), one
 *    power-of-two scale 2^e per 32 K elements stored as an E8M0 byte e + 127,
 *    e the smallest integer with max|v| <= 6 * 2^e (clamped to [-127, 127];
 *    an all-zero group has e = -127); codes round to nearest, ties to the
 *    even code, and a value that rounds to zero is encoded +0.  Two codes
 *    per byte; the even-K element is in the low nibble.
 *
 * Code matrices (activation codes, M rows; weight codes, N rows; K codes
 * per row) are stored in MFMA operand-block order: 1 KB blocks, each holding
 * the codes of 32 rows x 64 consecutive K values in the order the 64 lanes
 * of a 32x32x64 MFMA read them.  The byte holding codes (k, k + 1), k even,
 * of row i (for INT4: byte (k % 8) / 2 of the word that holds the eight
 * codes from k - k % 8 on) is at
 *     ((i / 32) * (K / 64) + k / 64) * 1024 + (i % 32 + 32 * ((k % 64) / 32)) * 16 + (k % 32) / 2
 * Rows are padded to a multiple of 32; the padding bytes are unspecified.
 *
 * FP4 scale matrices (E8M0 bytes, one per row and 32-wide group) follow the
 * same blocking: for each 32-row block and 128-wide K stage, 128 bytes; the
 * 2-byte slot of lane (i % 32) + 32 ((k / 32) % 2) holds the scales of the
 * stage's two 64-wide steps:
 *     ((i / 32) * (K / 128) + k / 128) * 128 + (i % 32 + 32 * ((k / 32) % 2)) * 2 + (k / 64) % 2
 * INT4 activation scales (fp16, one per row and 64-wide group) are blocked
 * the same way: for each 32-row block and 128-wide K stage, 128 bytes; the
 * 4-byte word of row i % 32 holds the stage's two groups:
 *     ((i / 32) * (K / 128) + k / 128) * 128 + (i % 32) * 4 + ((k / 64) % 2) * 2
 * INT4 weight scales are row-major [N][K / 64].
 *
 * bf16 low-rank matrices with `cols` columns (cols % 16 == 0: T, M x rank,
 * and L2 transposed, N x rank) are stored in 1 KB blocks of 32 rows x 16
 * columns in the lane order of a 32x32x16 bf16 MFMA; element (i, t) is at
 *     ((i / 32) * (cols / 16) + t / 16) * 512 + (i % 32 + 32 * ((t % 16) / 8)) * 8 + t % 8
 * (in elements), rows again padded to a multiple of 32.
 *
 * L1 transposed (rank x K bf16, the down-projection's operand) is stored in
 * 1 KB blocks in the lane order of a 16x16x32 bf16 MFMA: per 128-wide K chunk,
 * 16-row block and 8-wide step j = (k % 32) / 8; element (t, k) is at
 *     (((k / 128) * (rank / 16) + t / 16) * 4 + (k % 32) / 8) * 512
 *       + (t % 16 + 16 * ((k % 128) / 32)) * 8 + k % 8
 * (in elements). */
typedef enum svdq_format {
  SVDQ_INT4_G64_FP16 = 0,
  SVDQ_FP4_E2M1_G32_E8M0 = 1
} svdq_format;

typedef enum svdq_out_dtype {
  SVDQ_OUT_BF16 = 0,  /* Y stored as bf16 (round to nearest even) */
  SVDQ_OUT_F32 = 1    /* Y stored as fp32 */
} svdq_out_dtype;

enum {
  SVDQ_F_NO_SMOOTHING = 1u,  /* lambda = 1 (smoothing already folded into the previous op) */
  SVDQ_F_FACTORS_GIVEN = 2u, /* caller supplies L1, L2 instead of the SVD */
  SVDQ_F_HAS_BIAS = 4u       /* the layer has a bias vector b (N) */
};

/* One layer.  Supported: K % 128 == 0, 128 <= K <= 65536; N % 64 == 0,
 * 64 <= N <= 65536; rank % 16 == 0, 0 <= rank <= 128, rank <= min(K, N);
 * 0 <= alpha <= 1.  rank = 0 is plain per-group W4A4. */
typedef struct svdq_layer_desc {
  int32_t K;        /* input features */
  int32_t N;        /* output features */
  int32_t rank;     /* r, width of the low-rank branch */
  int32_t fmt;      /* svdq_format */
  float alpha;      /* smoothing migration strength (0.5 in the pages) */
  uint32_t flags;   /* SVDQ_F_* */
} svdq_layer_desc;

/* Text for a status code (static storage; never NULL). */
const char* svdq_status_string(int status);

/* Library version, as major * 10000 + minor * 100 + patch. */
int svdq_version(void);

/* Size in bytes of the prepared-weight blob for `desc`, or 0 if `desc` is
 * NULL or invalid.  The blob is position-independent (a 256-byte header with
 * byte offsets) and may be copied, saved and reloaded byte for byte. */
size_t svdq_prepared_bytes(const svdq_layer_desc* desc);

/* Device workspace that svdq_linear / svdq_linear_unfused need for M tokens:
 * the packed activation codes (ceil(M/32)*32 x K/2 bytes), the scales, the
 * bf16 down-projection (ceil(M/32)*32 x rank) and, for M <= 16384, room for
 * the fp32 partial down-projections of a K-split activation pass
 * (8 x M x rank x 4 bytes); for layers whose M x N output has few tiles
 * (INT4: at most 128 of 128 x 128; FP4: at most 32 of 256 x 256), a last,
 * optional 16 MiB for the fp32 partial tiles of a K-split GEMM (a workspace that ends before it is accepted and
 * runs the GEMM unsplit, so a workspace sized for a larger M still serves a
 * smaller one); 0 if arguments are invalid.  Every section is written
 * before it is read, so one workspace serves any layer and M. */
size_t svdq_workspace_bytes(const svdq_layer_desc* desc, int M, int unfused);

/* Byte sizes of svdq_quantize_act's three outputs for M tokens (codes,
 * scales, T).  Any output pointer may be NULL.  Returns SVDQ_OK or
 * SVDQ_ERR_INVALID_ARGUMENT / SVDQ_ERR_UNSUPPORTED_SHAPE. */
svdq_status svdq_act_sizes(const svdq_layer_desc* desc, int M, size_t* codes_bytes,
                           size_t* scales_bytes, size_t* t_bytes);

/* Calibration statistic for the smoothing factors (quantization handbook,
 * SmoothQuant section: lambda_j uses max_i |X_ij| over calibration
 * activations): d_absmax[j] = max_i |X[i, j]| over the M x K bf16 matrix
 * d_X.  With accumulate != 0 the result is max'ed into the existing
 * d_absmax (several calibration batches).  Asynchronous. */
svdq_status svdq_act_absmax(const void* d_X, int M, int K, float* d_absmax, int accumulate,
                            void* stream);

/* Offline preparation of one layer (walkthrough eq. (5); handbook
 * SmoothQuant and SVDQuant sections):
 *   lambda_j = a_j^alpha / w_j^(1-alpha), a = d_act_absmax, w_j = max_n |W[j,n]|
 *     (lambda = 1 where a_j or w_j is 0, or with SVDQ_F_NO_SMOOTHING);
 *     stored as fp32 lambda and fp32 1/lambda;
 *   W_hat = lambda * W (fp64); top-`rank` SVD W_hat ~ L1 L2 with
 *     L1 = U_r Sigma_r, L2 = V_r^T (randomized subspace iteration on the GPU
 *     with a Rayleigh-Ritz step), stored in bf16 - or, with
 *     SVDQ_F_FACTORS_GIVEN, the caller's d_L1 (K x r bf16) and d_L2
 *     (r x N bf16);
 *   R = W_hat - L1b L2b (fp64, summed over t in increasing order);
 *   R group-quantized along K for every output column, in `desc->fmt`, and
 *   packed into the blob's GEMM-native layout; bias (bf16, N) stored as fp32.
 * d_W: K x N bf16.  d_act_absmax: K fp32 (may be NULL only with
 * SVDQ_F_NO_SMOOTHING).  d_bias: N bf16, required iff SVDQ_F_HAS_BIAS.
 * d_prepared: device buffer of prepared_bytes >= svdq_prepared_bytes(desc).
 * Synchronous: returns after the blob is complete.  Allocates temporary
 * device memory (offline step). */
svdq_status svdq_prepare_weights(const svdq_layer_desc* desc, const void* d_W,
                                 const float* d_act_absmax, const void* d_bias,
                                 const void* d_L1, const void* d_L2, void* d_prepared,
                                 size_t prepared_bytes, void* stream);

/* svdq_prepare_weights with the residual quantized by GPTQ instead of
 * round-to-nearest (walkthrough, Table 3 row: GPTQ on the residual gives a
 * further gain).  H = x_hat^T x_hat of the calibration activations d_Xcal
 * (bf16, M_cal x K, x_hat = fp32(x * inv_lambda) as at run time), a channel
 * never active gets 1 on the diagonal, then damp * mean(diag H) is added to
 * the diagonal; U = upper Cholesky factor of H^-1 (H^-1 = U^T U).  The rows
 * k of R are quantized in increasing k; a group's scales (per output column)
 * are computed from the current rows when k reaches the group's first row,
 * with the same quantizer as round-to-nearest; the error of row k divided by
 * U[k][k] is taken off the rows i > k with weights U[k][i].  Same blob
 * format; a diagonal H gives the round-to-nearest blob exactly.  Synchronous;
 * allocates temporary device memory (x_hat, H, U: (M_cal + 2 K) K doubles)
 * and factors H on the host.  damp >= 0; SVDQ_ERR_INVALID_ARGUMENT also if H
 * is not positive definite. */
svdq_status svdq_prepare_weights_gptq(const svdq_layer_desc* desc, const void* d_W,
                                      const float* d_act_absmax, const void* d_bias,
                                      const void* d_L1, const void* d_L2, const void* d_Xcal,
                                      int M_cal, float damp, void* d_prepared,
                                      size_t prepared_bytes, void* stream);

/* An extra low-rank branch merged into the 16-bit branch of a prepared
 * layer, without touching the quantized residual (walkthrough, Fig. 9 and
 * Fig. 16 section: a LoRA runs as part of the low-rank branch, so a new
 * LoRA needs no re-quantization).  For an update dW = A B of the original
 * weight (d_A: K x r_extra, d_B: r_extra x N, bf16 row-major), X dW =
 * X_hat diag(lambda) A B, so the merged factors are
 *     L1' = [L1b | bf16(lambda32 (.) A)]   (row j scaled by lambda32_j; the
 *                                           fp64 product rounded once)
 *     L2' = [L2b ; B]
 * and lambda, inv_lambda, the residual codes and scales and the bias are
 * copied.  d_out receives the blob of the descriptor with rank
 * desc->rank + r_extra (format, K, N, alpha and flags unchanged), so
 * out_bytes >= svdq_prepared_bytes of that descriptor; d_out must not
 * overlap d_prepared.  r_extra > 0, r_extra % 16 == 0 and desc->rank +
 * r_extra <= 128, else SVDQ_ERR_UNSUPPORTED_SHAPE.  Synchronous.  Allocates
 * nothing. */
svdq_status svdq_merge_lowrank(const svdq_layer_desc* desc, const void* d_prepared, const void* d_A,
                               const void* d_B, int r_extra, void* d_out, size_t out_bytes, void* stream);

/* Reads the blob header back (synchronously) and checks it against `desc`:
 * magic, version, format, K, N, rank and flags.  SVDQ_ERR_BAD_BLOB if they
 * differ. */
svdq_status svdq_check_blob(const svdq_layer_desc* desc, const void* d_prepared, void* stream);

/* Fused activation pass (walkthrough Fig. 6, "down projection and
 * quantization share one input"; handbook timestep section: dynamic scales):
 *   x_hat = fp32(X * inv_lambda)                         (X: M x K bf16)
 *   per token row and K group: scale and 4-bit codes of x_hat in desc->fmt
 *     -> d_codes: ceil(M/32)*32 x K/2 bytes in MFMA operand-block order;
 *        d_scales: ceil(M/32)*32 x K/64 fp16 in the INT4 activation scale
 *        block order, or ceil(M/32)*32 x K/32 E8M0 bytes in the FP4 scale
 *        block order
 *   T = bf16(x_hat) L1b accumulated in fp32, rounded once to bf16
 *     -> d_T: ceil(M/32)*32 x rank bf16 in the bf16 block order (may be
 *        NULL when rank == 0).
 * Padding rows of the outputs are left unwritten.
 * X is read from HBM once.  `desc` must be the descriptor the blob was
 * prepared with.  d_workspace (optional, NULL allowed) is a buffer of
 * ws_bytes >= svdq_workspace_bytes(desc, M, 0) bytes, as svdq_linear takes:
 * with it, the pass may split K over several workgroups per row block and
 * add their fp32 partial T in a second kernel, in a fixed order (codes and
 * scales do not depend on the split; T is the same sum in another fp32
 * order, and is deterministic for a given device); without it, and with
 * rank > 0, each row block's T is accumulated by one workgroup.
 * Asynchronous. */
svdq_status svdq_quantize_act(const svdq_layer_desc* desc, const void* d_prepared,
                              const void* d_X, int M, void* d_codes, void* d_scales,
                              void* d_T, void* d_workspace, size_t ws_bytes, void* stream);

/* The fused layer: Y = Q(x_hat) Q(R) + Tb L2b + b, M x N in `out_dtype`.
 * Two kernels: the activation pass above (into d_workspace), then the 4-bit
 * GEMM whose K loop is followed by the rank-r bf16 K-slab Tb L2b in the same
 * fp32 accumulators and a bias epilogue (walkthrough Fig. 6: the
 * up-projection shares the 4-bit branch's output).  d_workspace must hold
 * svdq_workspace_bytes(desc, M, 0) bytes.  Asynchronous. */
svdq_status svdq_linear(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X,
                        int M, void* d_Y, int out_dtype, void* d_workspace, size_t ws_bytes,
                        void* stream);

/* Norm-fused activation pass: X is the input of the LayerNorm that precedes
 * the layer, and the smoothing is folded into that norm's affine (handbook,
 * SmoothQuant section: the smoothing factor is merged into the preceding
 * normalization's weights, so no separate operator runs):
 *   mu_i = mean_k x_ik,  rho_i = 1 / sqrt(mean_k (x_ik - mu_i)^2 + eps)
 *     (fp32 sums in a fixed order, one kernel)
 *   x_hat_ik = fma((x_ik - mu_i) rho_i, gamma'_k, beta'_k),
 *     gamma' = fp32(gamma * inv_lambda), beta' = fp32(beta * inv_lambda)
 * then the same quantization and down-projection as svdq_quantize_act, in
 * the same output layouts; x_hat is never written to memory.  d_gamma,
 * d_beta: bf16[K] (d_beta may be NULL: beta = 0); eps > 0 and finite.
 * d_workspace (svdq_workspace_bytes(desc, M, 0) bytes) is required: it holds
 * the row statistics and the folded affine.  Asynchronous. */
svdq_status svdq_quantize_act_ln(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X,
                                 const void* d_gamma, const void* d_beta, float eps, int M,
                                 void* d_codes, void* d_scales, void* d_T, void* d_workspace,
                                 size_t ws_bytes, void* stream);

/* The fused layer on the LayerNorm's input: svdq_linear with its activation
 * pass replaced by svdq_quantize_act_ln's (one extra launch for the row
 * statistics).  Y = Q(x_hat) Q(R) + Tb L2b + b with x_hat as above.
 * Asynchronous. */
svdq_status svdq_linear_ln(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X,
                           const void* d_gamma, const void* d_beta, float eps, int M, void* d_Y,
                           int out_dtype, void* d_workspace, size_t ws_bytes, void* stream);

/* The weight-only 4-bit layer (4-bit weights, 16-bit activations) for a few
 * token rows (diffusers page: the second operator, used for the
 * adaptive-norm and modulation projections next to the W4A4 layers):
 *   Y = round(x_hat dequant(Q(R)) + b),  x_hat = fp32(X * inv_lambda)
 * on a blob prepared with rank 0 (R = W_hat: the smoothed weight itself);
 * the activations are not quantized; accumulation in fp32 (deterministic
 * order).  M <= 16 and desc->rank == 0, else SVDQ_ERR_UNSUPPORTED_SHAPE.
 * d_workspace: svdq_workspace_bytes(desc, M, 0) bytes (partial outputs of a
 * K split).  Asynchronous. */
svdq_status svdq_linear_w4a16(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X,
                              int M, void* d_Y, int out_dtype, void* d_workspace, size_t ws_bytes,
                              void* stream);

/* The GEMM stage of svdq_linear on its own: Y = Q(x_hat) Q(R) + Tb L2b + b
 * from activations already produced by svdq_quantize_act with the same blob
 * (d_codes, d_scales, d_T in its output layouts; d_T may be NULL when
 * rank == 0).  svdq_linear is svdq_quantize_act followed by this call; the
 * split lets a caller time, overlap or reorder the two stages.
 * d_workspace (optional, NULL allowed): a buffer of ws_bytes >=
 * svdq_workspace_bytes(desc, M, 0) bytes; only its last section (the
 * partial tiles of a K-split INT4 GEMM) is used, so without it, or without
 * that section, the GEMM runs unsplit.  Asynchronous. */
svdq_status svdq_gemm(const svdq_layer_desc* desc, const void* d_prepared, const void* d_codes,
                      const void* d_scales, const void* d_T, int M, void* d_Y, int out_dtype,
                      void* d_workspace, size_t ws_bytes, void* stream);

/* The same layer computed the naive way, as separate kernels (walkthrough,
 * Nunchaku section: a separately run low-rank branch re-reads the 16-bit
 * activation and writes a 16-bit output again; Table 4's "SVDQuant" column):
 *   quantize (codes + scales only) -> down-projection (re-reads X, writes T)
 *   -> 4-bit GEMM + bias (writes Yp rounded to out_dtype)
 *   -> up-projection (reads Yp and T, writes Y = round(Yp + Tb L2b)).
 * Same arguments as svdq_linear; d_workspace holds
 * svdq_workspace_bytes(desc, M, 1) bytes.  Asynchronous. */
svdq_status svdq_linear_unfused(const svdq_layer_desc* desc, const void* d_prepared,
                                const void* d_X, int M, void* d_Y, int out_dtype,
                                void* d_workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fused
 * layer of svdq_linear without a workspace argument.  The activation codes,
 * scales, Tb and the partial down-projections go to a scratch array inside
 * the library, SVDQ_NOALLOC_SCRATCH_BYTES on each device it runs on, held
 * until the process ends.  The call allocates nothing: its first call on a
 * device looks up the array's device address once.
 *  - M is limited by the array: svdq_workspace_bytes(desc, M, 0) must not
 *    exceed SVDQ_NOALLOC_SCRATCH_BYTES, else SVDQ_ERR_BUFFER_TOO_SMALL and
 *    nothing is launched (64 MiB holds e.g. M = 16384 at K = 3072, M = 4608
 *    at K = 12288).
 *  - Every call on a device uses that device's one array, which keeps the
 *    last call's contents: calls that overlap on one device (different
 *    streams, or different threads without ordering) race on it and give
 *    wrong results.  Calls ordered on one stream are safe.
 * Other arguments, output and errors as svdq_linear.  Asynchronous. */
#define SVDQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
svdq_status svdq_linear_noalloc(const svdq_layer_desc* desc, const void* d_prepared, const void* d_X, int M,
                                void* d_Y, int out_dtype, void* stream);

/* Byte offsets of the blob's sections (for inspection, serialization and
 * tests).  All offsets are multiples of 256.
 *   lambda      fp32[K]
 *   inv_lambda  fp32[K]
 *   l1t         bf16, rank x K   (L1 transposed: row t holds column t of L1;
 *                                 L1 operand order)
 *   l2t         bf16, N x rank   (L2 transposed: row n holds column n of L2;
 *                                 bf16 block order)
 *   wcodes      u8, N x K/2      (residual codes of output column n as row n,
 *                                 in MFMA operand-block order)
 *   wscales     INT4: u16 fp16 bits [N][K/64] row-major; FP4: u8 E8M0,
 *               N x K/32 in the FP4 scale block order
 *   bias        fp32[N]          (offset 0 when the layer has no bias) */
typedef struct svdq_blob_layout {
  uint64_t header, lambda, inv_lambda, l1t, l2t, wcodes, wscales, bias, total;
} svdq_blob_layout;

svdq_status svdq_blob_layout_of(const svdq_layer_desc* desc, svdq_blob_layout* out);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
