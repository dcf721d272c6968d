/*
 * svdq.h -- C ABI of libsvdq, an MI355X (gfx950) implementation of the
 * SVDQuant W4A4 linear layer that replaces the large linears of a diffusion
 * transformer.
 *
 * The layer (aiflownews.com page, "What SVDQuant actually does" and "How
 * Nunchaku four bit quantization actually works"; t3chbillion.com page, the
 * W4A4 paragraph) computes
 *
 *     Y = X_hat L1 L2 + dequant(Q4(X_hat) Q4(R)) + b,   X_hat = X diag(lambda)^-1
 *
 * where lambda moves activation outliers into the weights, L1 L2 is a 16-bit
 * (bf16) low-rank branch from an SVD of the smoothed weight diag(lambda) W,
 * and R = diag(lambda) W - L1 L2 is the 4-bit residual. The pages say the
 * low-rank and 4-bit branches are fused so they share their input reads and
 * output writes (aiflownews.com, "Nunchaku: the inference engine that makes
 * SVDQuant practical"); here one kernel reads X once for smoothing, 4-bit
 * quantization and X_hat L1, and the 4-bit GEMM's epilogue adds (X_hat L1) L2
 * and b before the only write of Y.
 *
 * Formats ("SVDQuant supports both INT4 and FP4 data types", aiflownews.com):
 *   SVDQ_FMT_INT4_G64 : symmetric INT4 codes in [-7, 7] with an fp32 scale
 *                       max|v|/7 per 64 consecutive input channels (per token
 *                       for X, per output channel for R); codes are rounded
 *                       half-to-even from the exact quotient v/scale.
 *   SVDQ_FMT_MXFP4_G32: E2M1 codes with one E8M0 exponent per 32 consecutive
 *                       input channels (OCP MX: exponent = floor(log2 max|v|)-2,
 *                       elements rounded to nearest even, saturating at 6).
 *
 * Conventions for every entry point:
 *   - The caller owns and allocates every buffer. Host pointers are ordinary
 *     CPU memory; device pointers are HIP device memory (e.g. torch tensors).
 *   - Nothing is allocated, nothing is printed, no exception crosses the ABI.
 *     Every problem is returned as an svdq_status, checked before any launch.
 *   - GPU entry points enqueue work on `hip_stream` (a hipStream_t, NULL for
 *     the default stream) and return without synchronizing; buffers must stay
 *     alive until that stream has finished the work. The library keeps no
 *     pointer after returning.
 *   - Shapes: K % 256 == 0, N % 32 == 0, 0 <= rank <= 128 with rank % 16 == 0,
 *     rank <= min(K, N); M >= 0 (M == 0 is a no-op returning SVDQ_OK).
 *     K, N <= 65536; M <= 2^24; MXFP4 also (K + 128) * ceil(M / 32) < 2^31,
 *     INT4 also 32 * ceil(M / 32) * K <= 2^33 (activation codes of at most 4 GiB).
 *   - Device pointers (x, y, workspace and every packed buffer) must be
 *     16-byte aligned; a misaligned pointer returns SVDQ_ERR_SHAPE.
 *   - All functions are thread-safe; the only global state is a per-device
 *     cache of the "is this a gfx950 device" check. Two calls that share a
 *     workspace must be ordered (same stream or an event between them).
 *   - Environment: SVDQ_SYNC_DEBUG=1 synchronizes the stream after every
 *     launch and reports asynchronous faults as SVDQ_ERR_DEVICE;
 *     SVDQ_JACOBI_MAX_SWEEPS=n caps the pack's Jacobi sweeps (tests use 0 to
 *     exercise the non-convergence error).
 */
#ifndef SVDQ_H_
#define SVDQ_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SVDQ_API __attribute__((visibility("default")))
#else
#define SVDQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = 1,      /* a required pointer is NULL */
  SVDQ_ERR_SHAPE = 2,     /* K, N, rank, M (or a sub-window) outside the supported set */
  SVDQ_ERR_FORMAT = 3,    /* unknown svdq_format value */
  SVDQ_ERR_WORKSPACE = 4, /* workspace_bytes smaller than svdq_workspace_bytes() */
  SVDQ_ERR_NUMERIC = 5,   /* NaN/Inf in pack inputs, or the SVD iteration did not converge */
  SVDQ_ERR_DEVICE = 6     /* current device is not gfx950, or a HIP call/launch failed */
} svdq_status;

typedef enum { SVDQ_FMT_INT4_G64 = 0, SVDQ_FMT_MXFP4_G32 = 1 } svdq_format;

/* One layer: input channels K, output channels N, low-rank branch rank, format. */
typedef struct {
  int32_t K, N, rank, format;
} svdq_layer_desc;

/* Byte size of every buffer of a packed layer. */
typedef struct {
  size_t mu, l1, l2, qw, sw, bias;
} svdq_packed_sizes;

/*
 * A packed layer. The same struct describes the host copy written by the pack
 * calls and the device copy read by the forward call (copy each buffer
 * byte-for-byte to the device). Layouts are the library's own ("device
 * layout"); svdq_unpack_weights() returns the logical values.
 *   mu   fp32 [K]                 runtime smoothing multiplier mu_k = fl32(1/lambda_k)
 *   l1   bf16                     L1 [K][rank], rank padded to 32, shuffled for the MFMA
 *   bias bf16 [N]
 * Both formats, in MFMA fragment order (rows in blocks of 32; lane l = 32h + r
 * of a 64-lane fragment holds row 32b + r):
 *   qw   u8 [N/32][K/64][64][16]  lane 32h + r: 4-bit codes (INT4 two's
 *                                 complement or E2M1) of channels 64s + 32h +
 *                                 [0, 32), two per byte, low nibble first
 *   l2   bf16 [N/32][rank32/16][64][8]  L2 transposed, rank padded to a multiple
 *                                 of 32 (zeros); lane 32h + r of step c holds
 *                                 rank columns 16c + 8h + [0, 8)
 * Scales:
 *   sw   INT4:  fp32 [K/64][N]    per-group scales (group-major)
 *        MXFP4: u8 [K/128][N/32][64][2]  lane 32h + r of stage t: E8M0 bytes
 *                                 of the 32-channel blocks 4t + h and 4t + 2 + h
 */
typedef struct {
  float* mu;
  uint16_t* l1;
  uint16_t* l2;
  uint8_t* qw;
  void* sw;
  uint16_t* bias;
} svdq_packed;

/* Human-readable name of a status code (static storage, never NULL). */
SVDQ_API const char* svdq_status_string(svdq_status s);

/* Library version as an integer (major*10000 + minor*100 + patch). */
SVDQ_API int32_t svdq_version(void);

/*
 * Byte sizes of the packed buffers for `desc`. Host only.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT.
 */
SVDQ_API svdq_status svdq_packed_bytes(const svdq_layer_desc* desc, svdq_packed_sizes* out);

/*
 * Offline preparation of one layer, host only (the pages' "calibration,
 * quantization, packaging" step; aiflownews.com, "Deep integration with
 * Hugging Face Diffusers"):
 *   1. lambda_k = sqrt(act_absmax[k] / max_n |W[k,n]|) (1 where either is 0),
 *      mu_k = fl32(1/lambda_k); W_hat[k,n] = W[k,n] / mu_k in fp64;
 *   2. the top-`rank` singular triplets of W_hat by randomized subspace
 *      iteration seeded with `seed`; L1 = U_r Sigma_r, L2 = V_r^T, rounded
 *      to bf16;
 *   3. R = fl32(W_hat - L1 L2) (fp64, terms added in increasing rank index),
 *      quantized in `desc->format` per output channel.
 * w_lin: fp32 [N][K] (nn.Linear layout, W = w_lin^T). bias: fp32 [N] or NULL
 * (zeros). act_absmax: fp32 [K], max over calibration tokens of |X[:,k]|.
 * host_out: caller-allocated host buffers of svdq_packed_bytes() sizes.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT, SVDQ_ERR_NUMERIC
 * (non-finite input or an SVD that did not converge).
 */
SVDQ_API svdq_status svdq_pack_weights(const svdq_layer_desc* desc, const float* w_lin, const float* bias,
                              const float* act_absmax, uint64_t seed, svdq_packed* host_out);

/*
 * Step 3 of svdq_pack_weights alone, for given smoothing and factors (e.g.
 * factors computed elsewhere, or a LoRA-extended branch). Host only.
 * mu: fp32 [K]; l1: bf16 bits [K][rank]; l2: bf16 bits [rank][N] (logical,
 * row-major). The residual is taken against these bf16 factors.
 * Errors: as svdq_pack_weights.
 */
SVDQ_API svdq_status svdq_quantize_residual(const svdq_layer_desc* desc, const float* w_lin,
                                   const float* bias, const float* mu, const uint16_t* l1,
                                   const uint16_t* l2, svdq_packed* host_out);

/*
 * Logical view of a host packed layer (inverse of the device layout).
 * Any output pointer may be NULL to skip it.
 *   codes  int8 [N][K]: INT4 values in [-7,7], or E2M1 code bits 0..15
 *   scales INT4: fp32 [N][K/64]; MXFP4: u8 [N][K/32] (E8M0 bytes)
 *   l1 bf16 [K][rank]; l2 bf16 [rank][N]; bias bf16 [N]
 * Errors: SVDQ_ERR_NULL (desc/host), SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT.
 */
SVDQ_API svdq_status svdq_unpack_weights(const svdq_layer_desc* desc, const svdq_packed* host,
                                int8_t* codes, void* scales, uint16_t* l1, uint16_t* l2,
                                uint16_t* bias);

/*
 * Bytes of device workspace svdq_linear_forward needs for M tokens:
 * the 4-bit activation codes, their scales and the rank-32-padded
 * X_hat L1 product; INT4 layers add 32 MiB of GEMM scratch (fp32 partial
 * tiles and flags for the workgroups that share a tile's K stages, cleared
 * by svdq_stage1), and so do MXFP4 layers with M <= 256: with few tokens
 * the weight-streaming GEMM keeps its fp32 K-share partials there. With a low-rank branch, a last area holds kernel (1)'s
 * fp32 partial X_hat L1 per K piece (about twelve pieces) for up to 4096
 * rows, used when few token groups have their K pieces dealt over the CUs.
 * Host only.
 */
SVDQ_API svdq_status svdq_workspace_bytes(const svdq_layer_desc* desc, int64_t M, size_t* out);

/*
 * Runtime forward on the GPU: y = layer(x).
 *   x: bf16 [M][K] device, y: bf16 [M][N] device, dev: packed layer on the
 *   device, workspace: >= svdq_workspace_bytes(desc, M) device bytes (contents
 *   on entry are ignored; on return they hold the activation codes, scales
 *   and X_hat L1 of this call).
 * Two kernels on hip_stream: (1) smoothing + per-token 4-bit quantization +
 * X_hat L1 on bf16 MFMA from one read of X; (2) the 4-bit GEMM (INT8 MFMA
 * with int32 group sums and per-group dequant for INT4; block-scaled FP4
 * MFMA for MXFP4) whose epilogue adds (X_hat L1) L2 + b and writes bf16 Y.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT, SVDQ_ERR_WORKSPACE,
 * SVDQ_ERR_DEVICE (not gfx950 / launch failure).
 */
SVDQ_API svdq_status svdq_linear_forward(const svdq_layer_desc* desc, const svdq_packed* dev,
                                const uint16_t* x, int64_t M, uint16_t* y, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/*
 * Test hook: only kernel (1) of svdq_linear_forward, filling the workspace.
 * Same arguments and errors as svdq_linear_forward minus y.
 */
SVDQ_API svdq_status svdq_stage1(const svdq_layer_desc* desc, const svdq_packed* dev, const uint16_t* x,
                        int64_t M, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Kernel (2) of svdq_linear_forward alone: the 4-bit GEMM with its epilogue,
 * reading the activation codes, scales and X_hat L1 that svdq_stage1 left in
 * `workspace` for the same M. svdq_stage1 followed by svdq_gemm on one stream
 * equals svdq_linear_forward. Errors: as svdq_linear_forward.
 */
SVDQ_API svdq_status svdq_gemm(const svdq_layer_desc* desc, const svdq_packed* dev,
                               const void* workspace, size_t workspace_bytes, int64_t M,
                               uint16_t* y, void* hip_stream);

/*
 * Logical view of a workspace written by svdq_stage1/svdq_linear_forward and
 * copied to host memory. Any output may be NULL.
 *   codes int8 [M][K] (INT4 values or E2M1 code bits); scales INT4 fp32
 *   [M][K/64] or MXFP4 u8 [M][K/32]; z fp32 [M][rank] (bf16-rounded X_hat L1).
 */
SVDQ_API svdq_status svdq_unpack_workspace(const svdq_layer_desc* desc, int64_t M, const void* ws_host,
                                  size_t ws_bytes, int8_t* codes, void* scales, float* z);

/*
 * Test hook (INT4 only): the int32 group sums P[m][n][g] = sum over the 64
 * channels of group g of qx[m,k] qw[n,k] for the window m0 <= m < m0+mc,
 * n0 <= n < n0+nc, computed by the INT4 GEMM main loop (same kernel, an
 * epilogue that stores the raw per-group sums instead of dequantizing).
 * The workspace must hold svdq_stage1 output for M tokens.
 * p: int32 device [mc][nc][K/64]. Errors: as svdq_linear_forward.
 */
SVDQ_API svdq_status svdq_debug_int4_group_sums(const svdq_layer_desc* desc, const svdq_packed* dev,
                                       const void* workspace, size_t workspace_bytes, int64_t M,
                                       int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                       int32_t* p, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H_ */
