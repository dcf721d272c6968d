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
 * Formats (the pages give both a 4-bit integer and a 4-bit float variant;
 * aiflownews.com, "What SVDQuant actually does"):
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
 *   - Shapes: K % 64 == 0 (INT4) or K % 128 == 0 (MXFP4), N % 8 == 0,
 *     0 <= rank <= 128 with rank % 16 == 0, rank <= min(K, N); M >= 0 (M == 0
 *     is a no-op returning SVDQ_OK). K, N <= 65536; M <= 2^24. The packed
 *     layer and the workspace hold K padded to Kp = 256 ceil(K / 256) and N
 *     padded to Np = 32 ceil(N / 32) (the padding is zero and adds nothing);
 *     MXFP4 also (Kp + 128) * ceil(M / 32) < 2^31, INT4 also
 *     32 * ceil(M / 32) * Kp * 3 / 4 < 2^32 (the tiled GEMM's FP6 copy of the
 *     activation codes below 4 GiB).
 *   - Device pointers (x, y, workspace and every packed buffer) must be
 *     16-byte aligned; a misaligned pointer returns SVDQ_ERR_SHAPE.
 *   - All functions are thread-safe; the only global state is a per-device
 *     cache of the "is this a gfx950 device" check and, per device, the
 *     address of the array svdq_linear_forward_noalloc uses as its workspace.
 *     Two calls that share a workspace must be ordered (same stream or an
 *     event between them).
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
 * K and N below are the padded Kp and Np of the shape rules above (zeros in
 * the padding), except for mu.
 *   mu   fp32 [K]                 runtime smoothing multiplier mu_k = fl32(1/lambda_k)
 *                                 (the layer's K)
 *   l1   bf16                     L1 [K][rank], rank padded to 32, shuffled for the MFMA
 *   bias bf16 [N]
 * Both formats, in MFMA fragment order (rows in blocks of 32; lane l = 32h + r
 * of a 64-lane fragment holds row 32b + r):
 *   qw   u8 [N/32][K/64][64][16]  lane 32h + r: 4-bit codes (INT4 two's
 *                                 complement or E2M1) of channels 64s + 32h +
 *                                 [0, 32), two per byte, low nibble first;
 *                                 INT4 codes lie in [-7, 7] (the nibble 8,
 *                                 -8, is outside the format: the tiled GEMM's
 *                                 FP6 copy cannot hold it)
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
 * Offline preparation of one layer, host only (the offline calibrate, quantize
 * and package step of aiflownews.com, "Deep integration with Hugging Face
 * Diffusers"):
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
 * A LoRA adapter on a packed layer, without quantizing again (aiflownews.com,
 * "What SVDQuant actually does": pre-trained low-rank adapters work on the
 * 4-bit model as they are). Host only.
 * The adapter adds scale * X A B to the layer's output (A fp32 [K][lora_rank],
 * B fp32 [lora_rank][N], row-major; the usual LoRA down and up projections,
 * with scale = alpha / rank of the adapter). Since the layer sees X_hat =
 * X diag(mu), the adapter joins the 16-bit branch: the result is the layer of
 * rank base->rank + lora_rank with
 *   L1' = [L1 | bf16(A[k][i] * scale / mu_k)]  (fp64 multiply, then divide)
 *   L2' = [L2 ; bf16(B)]
 * and mu, the 4-bit codes and scales and the bias of `host_base` unchanged.
 * host_out->l1 and ->l2 must hold svdq_packed_bytes() of the extended
 * descriptor ({K, N, base->rank + lora_rank, format}). host_out->mu, ->qw, ->sw
 * and ->bias receive byte copies of the base's buffers, or may be NULL: the
 * extended layer can share the base's device buffers for them, so switching
 * adapters re-uploads only L1 and L2.
 * Errors: SVDQ_ERR_NULL; SVDQ_ERR_SHAPE (lora_rank <= 0, or the extended rank
 * outside the supported set: a multiple of 16, <= 128, <= min(K, N));
 * SVDQ_ERR_FORMAT; SVDQ_ERR_NUMERIC (non-finite adapter or scale, mu <= 0).
 */
SVDQ_API svdq_status svdq_lora_extend(const svdq_layer_desc* base, const svdq_packed* host_base,
                                      int32_t lora_rank, const float* lora_a, const float* lora_b,
                                      float scale, svdq_packed* host_out);

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
 * X_hat L1 product; INT4 layers add 64 MiB of GEMM scratch (fp32 partial
 * tiles and flags for the workgroups that share a tile's K stages, cleared
 * by svdq_stage1), and so do MXFP4 layers with M <= 256: with few tokens
 * the weight-streaming GEMM keeps its fp32 K-share partials there. With a
 * low-rank branch, an area holds kernel (1)'s fp32 partial X_hat L1 per K
 * piece (about twelve pieces) for up to 4096 rows, used when few token
 * groups have their K pieces dealt over the CUs. INT4 layers with M > 256
 * end with the tiled GEMM's FP6 copies of the activation and weight codes
 * (3/4 byte per code: 32 ceil(M / 32) Kp and Np Kp codes), which every
 * GEMM refills from the 4-bit codes. Host only.
 */
SVDQ_API svdq_status svdq_workspace_bytes(const svdq_layer_desc* desc, int64_t M, size_t* out);

/*
 * Runtime forward on the GPU: y = layer(x).
 *   x: bf16 [M][K] device, y: bf16 [M][N] device, dev: packed layer on the
 *   device, workspace: >= svdq_workspace_bytes(desc, M) device bytes (contents
 *   on entry are ignored; on return they hold the activation codes, scales
 *   and X_hat L1 of this call).
 * Kernels on hip_stream: (1) smoothing + per-token 4-bit quantization +
 * X_hat L1 on bf16 MFMA from one read of X; (2) the 4-bit GEMM (for INT4,
 * exact per-group sums and per-group dequant: on FP6 copies of the codes
 * that a small kernel writes into the workspace first with more than 256
 * tokens, on INT8 MFMA with fewer; block-scaled FP4 MFMA for MXFP4) whose
 * epilogue adds (X_hat L1) L2 + b and writes bf16 Y.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT, SVDQ_ERR_WORKSPACE,
 * SVDQ_ERR_DEVICE (not gfx950 / launch failure).
 */
SVDQ_API svdq_status svdq_linear_forward(const svdq_layer_desc* desc, const svdq_packed* dev,
                                const uint16_t* x, int64_t M, uint16_t* y, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/*
 * svdq_linear_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same kernels and result as svdq_linear_forward; the workspace is
 * a device array the library owns, SVDQ_NOALLOC_SCRATCH_BYTES (256 MiB) per
 * GPU, set aside when the library first runs on that GPU and held until the
 * process ends. Nothing is allocated here, and M is limited to the M for which
 * svdq_workspace_bytes(desc, M) <= SVDQ_NOALLOC_SCRATCH_BYTES (every linear of
 * a FLUX transformer block at up to 4608 tokens; the largest, K = 15360 and
 * N = 3072, needs 211 MiB). Every call on one GPU uses the same
 * array and leaves this call's codes, scales and X_hat L1 in it: calls that
 * overlap on one GPU (two streams, or two host threads without ordering)
 * race and give wrong results, so order them.
 * Errors: as svdq_linear_forward; SVDQ_ERR_WORKSPACE when the workspace for M
 * exceeds the array.
 */
#define SVDQ_NOALLOC_SCRATCH_BYTES (256u << 20)
SVDQ_API svdq_status svdq_linear_forward_noalloc(const svdq_layer_desc* desc, const svdq_packed* dev,
                                                 const uint16_t* x, int64_t M, uint16_t* y, void* hip_stream);

/*
 * The MLP of a transformer block on the 4-bit path: y = down(GELU(up(x))),
 * GELU(v) = v Phi(v) (Phi the standard normal distribution function),
 * applied to the bf16 output of `up` and rounded to bf16, as a separate
 * activation between the two layers would be. The engine that runs SVDQuant
 * fuses kernels that work on the same data, to cut memory traffic
 * (aiflownews.com, "Nunchaku: the inference engine that makes SVDQuant
 * practical"); here the up layer's GEMM epilogue applies the GELU and emits
 * the down layer's kernel-(1) output directly: its smoothed 4-bit codes and
 * scales (INT4 or MXFP4, the pair's format) and, per tile column of hidden
 * channels, the partial X_hat L1, which one small kernel adds up. The hidden
 * activation never goes to memory.
 *   up: K0 -> N0, down: N0 -> N1 (down->K == up->N); x bf16 [M][K0],
 *   y bf16 [M][N1] (device, 16-byte aligned); dev_up, dev_down: packed
 *   layers on the device; workspace: >= svdq_mlp_workspace_bytes device
 *   bytes; contents on entry ignored, on return the down layer's part (from
 *   *down_offset) holds its codes, scales and X_hat L1 as svdq_stage1 lays
 *   them out, for rows below M (the fused path leaves rows M .. round32(M)
 *   as the composition leaves them: unwritten by this call).
 *   mode SVDQ_MLP_AUTO: fused when svdq_mlp_fused says so, else the
 *   composition; SVDQ_MLP_UNFUSED: always the composition (svdq_linear_forward
 *   of up into the workspace, a GELU kernel in place, svdq_linear_forward of
 *   down; the bf16 hidden activation [M][up N] is left in the workspace at
 *   *down_offset plus the down layer's svdq_workspace_bytes rounded up to a
 *   multiple of 256). The fused path's codes and scales equal the composition's bit for
 *   bit (same GELU, same quantizer); its Z differs only in the fp32 summation
 *   order of the partial X_hat L1.
 * Fused when both layers have the same format, up->N is a whole number of
 * the tiled GEMM's tile columns (256 channels INT4, 384 MXFP4) and of 256,
 * M > 256 (the
 * tiled GEMM; fewer tokens take the weight-streaming kernel, with no fused
 * epilogue) and the partial X_hat L1, (up->N / tile width) M
 * rank32(down->rank) fp32 values, stays below 4 GiB. Errors: as svdq_linear_forward for either layer; SVDQ_ERR_SHAPE
 * also for down->K != up->N or an unknown mode.
 * svdq_mlp_workspace_bytes: the workspace bytes for M tokens and (if
 * down_offset is not NULL) where the down layer's part starts in it.
 * svdq_mlp_fused: *fused = 1 when SVDQ_MLP_AUTO takes the fused path for M.
 * Both host only; errors SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_FORMAT.
 */
#define SVDQ_MLP_AUTO 0
#define SVDQ_MLP_UNFUSED 1
SVDQ_API svdq_status svdq_mlp_workspace_bytes(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M,
                                              size_t* out, size_t* down_offset);
SVDQ_API svdq_status svdq_mlp_fused(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M,
                                    int32_t* fused);
SVDQ_API svdq_status svdq_mlp_forward(const svdq_layer_desc* up, const svdq_packed* dev_up,
                                      const svdq_layer_desc* down, const svdq_packed* dev_down, const uint16_t* x,
                                      int64_t M, uint16_t* y, void* workspace, size_t workspace_bytes, int32_t mode,
                                      void* hip_stream);

/*
 * Test hook: only kernel (1) of svdq_linear_forward, filling the workspace.
 * Same arguments and errors as svdq_linear_forward minus y.
 */
SVDQ_API svdq_status svdq_stage1(const svdq_layer_desc* desc, const svdq_packed* dev, const uint16_t* x,
                        int64_t M, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Kernel (1) with its outputs in logical layouts on the device: the smoothed
 * activations' 4-bit codes and scales and the low-rank product X_hat L1
 * (aiflownews.com, "What SVDQuant actually does": smoothing, the 16-bit
 * low-rank branch, 4-bit activations). Runs svdq_stage1 on the workspace
 * (which it leaves filled), then one small kernel on the same stream writes
 *   codes  int8 [M][K]: INT4 values in [-7,7], or E2M1 code bits 0..15
 *   scales INT4: fp32 [M][K/64]; MXFP4: u8 [M][K/32] (E8M0 bytes)
 *   z      fp32 [M][rank]: X_hat L1 as the GEMM uses it (bf16 values)
 * Device pointers, each may be NULL to skip it; z and INT4 scales 4-byte
 * aligned. Nothing is allocated.
 * Errors: as svdq_stage1; SVDQ_ERR_SHAPE for a misaligned fp32 output.
 */
SVDQ_API svdq_status svdq_stage1_outputs(const svdq_layer_desc* desc, const svdq_packed* dev, const uint16_t* x,
                                         int64_t M, int8_t* codes, void* scales, float* z, void* workspace,
                                         size_t workspace_bytes, void* hip_stream);

/*
 * Kernel (2) of svdq_linear_forward alone: the 4-bit GEMM with its epilogue
 * (for INT4 with more than 256 tokens, preceded by the kernel that writes the
 * FP6 copies of the codes into the workspace), reading the activation codes,
 * scales and X_hat L1 that svdq_stage1 left in `workspace` for the same M.
 * svdq_stage1 followed by svdq_gemm on one stream equals svdq_linear_forward.
 * Errors: as svdq_linear_forward.
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
 * n0 <= n < n0+nc. They come from the GEMM kernel svdq_linear_forward runs
 * for this M (the same dispatch): the tiled kernel, over the window's tiles
 * as whole tiles, or with few tokens the weight-streaming kernel in the
 * forward's own launch shape (K shares, K parts, token parts). Both use the
 * forward's operands and MFMAs (the tiled kernel's FP6 copies of the codes
 * and block-scaled MFMAs, the few-token kernel's widened nibbles and i8
 * MFMAs) and store each group's sum instead of dequantizing it. Only entries inside the window are written.
 * The workspace must hold svdq_stage1 output for M tokens.
 * p: int32 device [mc][nc][K/64]. Errors: as svdq_linear_forward.
 */
SVDQ_API svdq_status svdq_debug_int4_group_sums(const svdq_layer_desc* desc, const svdq_packed* dev,
                                       const void* workspace, size_t workspace_bytes, int64_t M,
                                       int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                                       int32_t* p, void* hip_stream);

/*
 * GPU-side pack (the calibrate-quantize-package step on the device; the pages'
 * offline workflow, aiflownews.com, "Native Diffusers integration and the new
 * workflow"): the steps of svdq_pack_weights with the column maxima, the
 * randomized SVD's products with W_hat, the residual and its quantization on
 * the GPU (the panel orthonormalizations and the small Jacobi SVD on the
 * host). The smoothing has strength alpha: lambda_k = ax_k^alpha /
 * aw_k^(1 - alpha) (fp64; at alpha = 0.5 computed as sqrt(ax / aw), which is
 * svdq_pack_weights' rule; 1 where either maximum is 0). Given the same mu and
 * bf16 factors the codes and scales are the host pack's bits.
 * w_lin fp32 [N][K], bias fp32 [N] or NULL, act_absmax fp32 [K]: DEVICE
 * pointers. dev_out: device buffers of svdq_packed_bytes() sizes. workspace:
 * >= svdq_pack_gpu_workspace_bytes() device bytes. Runs on hip_stream and
 * synchronizes it (host steps in between); not for graph capture.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE (also alpha outside [0, 1]),
 * SVDQ_ERR_FORMAT, SVDQ_ERR_WORKSPACE, SVDQ_ERR_NUMERIC, SVDQ_ERR_DEVICE.
 */
SVDQ_API svdq_status svdq_pack_gpu_workspace_bytes(const svdq_layer_desc* desc, size_t* out);
SVDQ_API svdq_status svdq_pack_weights_gpu(const svdq_layer_desc* desc, const float* w_lin, const float* bias,
                                           const float* act_absmax, float alpha, uint64_t seed,
                                           svdq_packed* dev_out, void* workspace, size_t workspace_bytes,
                                           void* hip_stream);

/*
 * Calibrated smoothing strength (aiflownews.com, "What SVDQuant actually
 * does": a calibration pass on representative data): for each alpha of
 * alphas[n_alpha] (host, each in [0, 1], at most 64) the layer is packed on
 * the GPU as svdq_pack_weights_gpu does (act_absmax = max over the
 * calibration rows) and run on the calibration rows x_cal (bf16 [m_cal][K],
 * device); the loss is the squared error of its bf16 output against
 * x_cal W^T + b (fp64). The first alpha of least loss is kept: dev_out holds
 * that layer, *alpha_out (may be NULL) its alpha, losses_out (host
 * [n_alpha], may be NULL) every loss. workspace: >=
 * svdq_calibrate_workspace_bytes(desc, m_cal). Synchronizes hip_stream.
 * Errors: as svdq_pack_weights_gpu, and SVDQ_ERR_SHAPE for m_cal outside
 * 1..65536 or n_alpha outside 1..64.
 */
SVDQ_API svdq_status svdq_calibrate_workspace_bytes(const svdq_layer_desc* desc, int64_t m_cal, size_t* out);
SVDQ_API svdq_status svdq_calibrate_alpha(const svdq_layer_desc* desc, const float* w_lin, const float* bias,
                                          const uint16_t* x_cal, int64_t m_cal, const float* alphas,
                                          int32_t n_alpha, uint64_t seed, float* alpha_out, double* losses_out,
                                          svdq_packed* dev_out, void* workspace, size_t workspace_bytes,
                                          void* hip_stream);

/*
 * ---------------------------------------------------------------------------
 * AWQ-style W4A16 linear: 4-bit weights, 16-bit activations, for the
 * adaptive-normalization and modulation layers the pages keep at higher
 * precision (aiflownews.com, "How Nunchaku four bit quantization actually
 * works"). y = x diag(inv_s) dequant(Q)^T + b with inv_s = fl32(1/s), s the
 * activation-aware channel scales, and Q the 4-bit codes of W diag(s):
 * per output channel and group of 128 input channels an fp32 scale and a
 * u8 zero point, w = scale * (q - zero) with q in [0, 15].
 * Shapes: K % 128 == 0, K <= 4096, N % 16 == 0, N <= 65536; M >= 0.
 * Device layout (the host copy written by svdq_awq_pack, copied byte for byte):
 *   inv_s  fp32 [K]
 *   qw     u8 [N/16][K/128][64][16]: lane l = 16c + r holds output row 16b + r;
 *          its 4-byte word t holds channels 128g + 32t + 8c + (0..7), element
 *          2i in bits 4i..4i+3 and element 2i+1 in bits 16+4i..16+4i+3
 *   scales fp32 [N/16][K/128][16], zeros u8 [N/16][K/128][16]  (row 16b + r at r)
 *   bias   bf16 [N]
 * ---------------------------------------------------------------------------
 */
typedef struct {
  int32_t K, N;
} svdq_awq_desc;

typedef struct {
  size_t inv_s, qw, scales, zeros, bias;
} svdq_awq_sizes;

typedef struct {
  float* inv_s;
  uint8_t* qw;
  float* scales;
  uint8_t* zeros;
  uint16_t* bias;
} svdq_awq_packed;

/* Byte sizes of the buffers of an AWQ layer. Host only.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE. */
SVDQ_API svdq_status svdq_awq_packed_bytes(const svdq_awq_desc* desc, svdq_awq_sizes* out);

/*
 * Offline preparation of an AWQ layer, host only. a_k = mean over the m_cal
 * calibration rows x_cal (fp32 [m_cal][K]) of |x_cal[m,k]|; for alpha on the
 * grid 0, 1/20, ..., 19/20 (or `alpha` when it is in [0, 1]; a negative value
 * searches): s_k = max(a_k, 1e-4)^alpha / sqrt(max s * min s), W diag(s)
 * quantized per group as above (fp32: scale = max(max - min, 1e-5) / 15,
 * zero = clamp(-rint(min / scale), 0, 15), q = clamp(rint(w / scale) + zero,
 * 0, 15)), and the candidate's loss the squared error of its output against
 * x_cal W^T; the first alpha of least loss is kept.
 * w_lin fp32 [N][K]; bias fp32 [N] or NULL. alpha_out and s_out (fp64 [K],
 * the chosen s) may be NULL. host_out: buffers of svdq_awq_packed_bytes().
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE (also m_cal <= 0, alpha > 1),
 * SVDQ_ERR_NUMERIC (non-finite input).
 */
SVDQ_API svdq_status svdq_awq_pack(const svdq_awq_desc* desc, const float* w_lin, const float* bias,
                                   const float* x_cal, int64_t m_cal, float alpha, double* alpha_out,
                                   double* s_out, svdq_awq_packed* host_out);

/* Logical view of a host AWQ layer: codes u8 [N][K] (0..15), scales fp32
 * [N][K/128], zeros u8 [N][K/128]; any output may be NULL. */
SVDQ_API svdq_status svdq_awq_unpack(const svdq_awq_desc* desc, const svdq_awq_packed* host, uint8_t* codes,
                                     float* scales, uint8_t* zeros);

/*
 * Runtime forward on the GPU: y bf16 [M][N] = layer(x bf16 [M][K]), one
 * kernel on hip_stream. x_hat = fl32(x inv_s) is rounded to bf16 for the
 * bf16 MFMA; sums in fp32, in an order fixed by K alone, so a row's output
 * is the same bits whatever M and the other rows are. Built for a few rows
 * (it streams the weights once per 16 rows). No workspace, nothing
 * allocated. Device pointers 16-byte aligned. Errors: SVDQ_ERR_NULL,
 * SVDQ_ERR_SHAPE, SVDQ_ERR_DEVICE.
 */
SVDQ_API svdq_status svdq_awq_forward(const svdq_awq_desc* desc, const svdq_awq_packed* dev, const uint16_t* x,
                                      int64_t M, uint16_t* y, void* hip_stream);

/*
 * Measured ceilings of the GPU (not part of the layer; the benchmark reports
 * the kernels against them beside the published peaks).
 * svdq_measure_mfma_peak enqueues one MFMA-only loop on every compute unit:
 * kind 0 v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands (the MXFP4 GEMM's
 * instruction), 1 v_mfma_i32_32x32x32_i8 (the INT4 GEMM's), 2
 * v_mfma_f32_32x32x16_bf16 (the low-rank branch's), `iters` steps of four
 * independent accumulators per wave, operand bits random per lane or, with
 * constant_operands, one fixed pattern. *flops receives the loop's operation
 * count (2 per multiply-add); time it with events on hip_stream.
 * Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE (kind outside 0..2, iters outside
 * 1..2^24), SVDQ_ERR_DEVICE.
 */
SVDQ_API svdq_status svdq_measure_mfma_peak(int32_t kind, int32_t constant_operands, int32_t iters,
                                            double* flops, void* hip_stream);

/*
 * Enqueues dst = src for `bytes` device bytes (16-byte loads and stores over
 * eight workgroups per compute unit): 2 * bytes of HBM traffic when neither
 * buffer fits the caches. Both pointers 16-byte aligned, bytes % 16 == 0, the
 * buffers must not overlap. Errors: SVDQ_ERR_NULL, SVDQ_ERR_SHAPE, SVDQ_ERR_DEVICE.
 */
SVDQ_API svdq_status svdq_measure_copy(const void* src, void* dst, size_t bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H_ */
