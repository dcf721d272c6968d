"""CPU oracle for the SVDQuant W4A4 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package's smoke check and the benchmark's CPU
baseline may import this module. The product (the HIP library and its Python
binding) never calls it, and this module imports nothing from the product.

What it computes, in the pages' order ("What SVDQuant actually does" and
"How Nunchaku four bit quantization actually works", aiflownews.com page;
the W4A4 description on the t3chbillion.com page):

  pack (offline):
    1. move activation outliers into the weights: per input channel k a
       smoothing factor lambda_k; the layer keeps mu_k = fl32(1/lambda_k) and
       the runtime multiplies X by mu (so X_hat = X diag(lambda)^-1) while
       the weight rows are divided by mu (W_hat = diag(lambda) W);
    2. SVD of W_hat; the top-r part, kept in 16 bit (bf16), is the low-rank
       branch L1 [K][r] = U_r Sigma_r, L2 [r][N] = V_r^T;
    3. the residual R = W_hat - L1 L2 (taken against the bf16 factors) is
       quantized to 4 bits: INT4 per output channel per group of 64 input
       channels, or MXFP4 (E2M1 values with an E8M0 scale per 32).
  forward (runtime):
    X_hat = X * mu; Q4(X_hat) per token per group (64 for INT4, 32 for
    MXFP4); Y = X_hat L1 L2 + dequant(Q4(X_hat) Q4(R)) + b.

Precision: every quantity that decides an integer code is computed in the
precision the method defines (fp32 smoothed activations and scales, the
exact quotient for rounding); sums that form Y are taken in float64.

Readings of points the pages leave open are the ones listed in the project's
design notes (lambda = sqrt(max|X|/max|W|), Sigma folded into L1, bf16
factors, residual against the rounded factors, fp32 INT4 scales amax/7,
round-half-to-even of the exact quotient, codes in [-7, 7], OCP MX E8M0
exponent floor(log2 amax) - 2, sign kept on E2M1 zeros).

Every function here is pinned by tests/test_oracle.py against brute force,
closed forms and invariants; none is "parity unpinned".

A packed layer can also take a LoRA adapter without re-quantization
(lora_extend): the adapter joins the 16-bit low-rank branch and the 4-bit
residual is kept (same page, same section).

Two layers in a row with a GELU between (a transformer block's MLP,
mlp_forward): the engine fuses kernels that work on the same data ("Nunchaku:
the inference engine that makes SVDQuant practical", aiflownews.com page).
Fusion changes no value, so the oracle is the plain composition: the up
layer's output as bf16, GELU, bf16, the down layer.
"""
from __future__ import annotations

import math

import numpy as np

GROUP_INT4 = 64
BLOCK_MX = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # index == code bits e|m


# ----------------------------------------------------------------------------
# bf16 helpers (round to nearest even), written out from the bf16 definition:
# bf16 keeps the top 16 bits of the IEEE binary32 pattern.
# ----------------------------------------------------------------------------
def to_bf16(a) -> np.ndarray:
    """Round real values (float64 or float32) to the nearest bf16, ties to even,
    in one rounding; returns float32 holding the bf16 value. bf16 has float32's
    exponent range with 7 fraction bits: 8 significant bits down to 2^-126, then
    gradual underflow with a fixed spacing of 2^-133 (the subnormals).
    v = f * 2^E with f in [0.5, 1): the spacing is 2^q with q = max(E - 8, -133),
    and bf16(v) = rint(v / 2^q) * 2^q, exact in float64 (values past the largest
    bf16 by half a spacing become inf in the float32 cast)."""
    v = np.asarray(a, dtype=np.float64)
    _, E = np.frexp(v)
    q = np.maximum(E.astype(np.float64) - 8.0, -133.0)
    return (np.rint(v * np.exp2(-q)) * np.exp2(q)).astype(np.float32)


def bf16_from_bits(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_to_bits(vals_f32) -> np.ndarray:
    return (np.asarray(vals_f32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# Step 1: smoothing ("shift activation outliers into the weights")
# ----------------------------------------------------------------------------
def smoothing_factors(act_absmax: np.ndarray, w_lin: np.ndarray):
    """lambda_k = sqrt(max_m|X[m,k]| / max_n|W[k,n]|) in float64, 1 where either max is 0.

    Returns (lam float64 [K], mu float32 [K]) with mu = fl32(1/lam).
    """
    ax = np.asarray(act_absmax, dtype=np.float32).astype(np.float64)
    aw = np.abs(np.asarray(w_lin, dtype=np.float32)).max(axis=0).astype(np.float64)
    lam = np.ones_like(ax)
    ok = (ax > 0) & (aw > 0)
    lam[ok] = np.sqrt(ax[ok] / aw[ok])
    mu = (1.0 / lam).astype(np.float32)
    return lam, mu


def smoothing_factors_alpha(act_absmax: np.ndarray, w_lin: np.ndarray, alpha: float):
    """Smoothing of strength alpha: lambda_k = ax_k^alpha / aw_k^(1 - alpha)
    (float64; 1 where either maximum is 0), mu = fl32(1 / lambda). At alpha =
    1/2 this is the default rule and is computed as it is, sqrt(ax / aw).
    Returns (lam float64 [K], mu float32 [K])."""
    if alpha == 0.5:
        return smoothing_factors(act_absmax, w_lin)
    ax = np.asarray(act_absmax, dtype=np.float32).astype(np.float64)
    aw = np.abs(np.asarray(w_lin, dtype=np.float32)).max(axis=0).astype(np.float64)
    lam = np.ones_like(ax)
    ok = (ax > 0) & (aw > 0)
    lam[ok] = np.power(ax[ok], alpha) / np.power(aw[ok], 1.0 - alpha)
    return lam, (1.0 / lam).astype(np.float32)


def calibrate_alpha(w_lin, bias, x_cal, rank: int, fmt: str, alphas) -> dict:
    """Calibrated smoothing strength (aiflownews.com, "What SVDQuant actually
    does": the method is calibrated on representative data before it is
    quantized): for each alpha the whole pack (smoothing of strength alpha,
    SVD, residual, quantization) and the layer's output on the calibration
    rows; the loss is the squared error against x W^T + b, and the first
    alpha of least loss is kept. Returns dict(alpha, losses, packed)."""
    w_lin = np.asarray(w_lin, np.float32)
    x = np.asarray(x_cal, np.float32)
    ax = np.abs(x).max(axis=0)
    ref = x.astype(np.float64) @ w_lin.T.astype(np.float64)
    if bias is not None:
        ref = ref + np.asarray(bias, np.float32).astype(np.float64)[None, :]
    losses, packs = [], []
    for al in alphas:
        _, mu = smoothing_factors_alpha(ax, w_lin, float(al))
        w_hat = smoothed_weight(w_lin, mu)
        l1, l2 = low_rank_factors(w_hat, rank)
        p = pack(w_lin, bias, ax, rank, fmt, factors=(mu, l1, l2))
        losses.append(float(np.sum((forward(p, x) - ref) ** 2)))
        packs.append(p)
    i = int(np.argmin(losses))
    return dict(alpha=float(alphas[i]), losses=np.array(losses), packed=packs[i])


def smoothed_weight(w_lin: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """W_hat [K][N] float64, W_hat[k,n] = W[k,n] / mu_k (the exact inverse of the runtime multiply)."""
    w = np.asarray(w_lin, dtype=np.float32).astype(np.float64).T  # math layout K x N
    return w / np.asarray(mu, dtype=np.float32).astype(np.float64)[:, None]


def smooth_activations(x: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """X_hat = fl32(x * mu_k), one float32 multiply per element."""
    return np.asarray(x, dtype=np.float32) * np.asarray(mu, dtype=np.float32)[None, :]


# ----------------------------------------------------------------------------
# Step 2: the 16-bit low-rank branch from an SVD of the smoothed weight
# ----------------------------------------------------------------------------
def low_rank_factors(w_hat: np.ndarray, rank: int, round_bf16: bool = True):
    """L1 = U_r Sigma_r [K][r], L2 = V_r^T [r][N] from a full SVD of W_hat (float64).

    With ``round_bf16`` the factors are rounded to bf16 (returned as float32
    arrays holding bf16 values); otherwise they are returned in float64.
    """
    K, N = w_hat.shape
    if rank == 0:
        z1, z2 = np.zeros((K, 0)), np.zeros((0, N))
        return (z1.astype(np.float32), z2.astype(np.float32)) if round_bf16 else (z1, z2)
    u, s, vt = np.linalg.svd(w_hat, full_matrices=False)
    l1 = u[:, :rank] * s[None, :rank]
    l2 = vt[:rank, :]
    if round_bf16:
        return to_bf16(l1), to_bf16(l2)
    return l1, l2


def residual(w_hat: np.ndarray, l1: np.ndarray, l2: np.ndarray) -> np.ndarray:
    """R = fl32(W_hat - sum_i L1[:,i] L2[i,:]), the sum taken in float64 in increasing i,
    one multiply then one add per term (no fused multiply-add)."""
    acc = np.zeros_like(w_hat, dtype=np.float64)
    l1d = np.asarray(l1, dtype=np.float64)
    l2d = np.asarray(l2, dtype=np.float64)
    for i in range(l1d.shape[1]):
        prod = l1d[:, i:i + 1] * l2d[i:i + 1, :]
        acc = acc + prod
    return (w_hat - acc).astype(np.float32)


# ----------------------------------------------------------------------------
# Step 3: 4-bit quantizers
# ----------------------------------------------------------------------------
def quant_int4_rows(v: np.ndarray, group: int = GROUP_INT4):
    """Symmetric INT4 along the last axis, per group of ``group`` elements.

    s = fl32(max|v| / 7) (an IEEE float32 divide), q = round-half-to-even of
    the exact quotient v/s, clamped to [-7, 7]; a group whose max is 0 gets
    s = 0 and q = 0. Returns (q int8 same shape, s float32 [..., L/group]).
    The float64 quotient of two float32 numbers is on the correct side of
    every half-integer (it is exact at a tie and its error is far below the
    smallest possible non-tie distance), so rint of it is the exact RNE.
    """
    v = np.asarray(v, dtype=np.float32)
    *lead, L = v.shape
    assert L % group == 0
    g = v.reshape(*lead, L // group, group)
    amax = np.abs(g).max(axis=-1)
    s = (amax / np.float32(7.0)).astype(np.float32)
    sd = s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sd > 0, np.rint(g.astype(np.float64) / np.where(sd > 0, sd, 1.0)), 0.0)
    q = np.clip(q, -7, 7).astype(np.int8)
    return q.reshape(*lead, L), s


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """OCP MX shared exponent for E2M1 elements: floor(log2 amax) - 2 (2 = E2M1's
    largest exponent), clamped to [-127, 127]; amax == 0 gives -127.
    floor(log2) is read off frexp (amax = f * 2^E, f in [0.5, 1) -> E - 1)."""
    amax = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, E = np.frexp(amax)
    e = np.where(amax > 0, (E - 1) - 2, -127)
    return np.clip(e, -127, 127).astype(np.int32)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """E2M1 code (4 bits: sign|e1 e0|m) of real values v, round to nearest with
    ties to the even mantissa bit, saturating at 6. The sign bit is the sign
    of v (a negative value that rounds to zero keeps its sign bit)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    d = np.abs(a[..., None] - E2M1_GRID)            # distance to every grid point
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin                                  # one or two nearest points
    idx = np.arange(8)
    # among the nearest points, prefer the even code (mantissa bit 0)
    score = np.where(cand, (idx & 1) * 16 + idx, 1 << 10)
    code = score.argmin(axis=-1)
    code = np.where(a > 6.0, 7, code)
    sign = np.signbit(v).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    """Value of E2M1 codes from the bit fields (exponent bias 1, one mantissa bit)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.exp2(e - 1.0))
    return s * mag


def quant_mxfp4_rows(v: np.ndarray, block: int = BLOCK_MX):
    """MXFP4 along the last axis: per block of 32, e = e8m0_exponent(max|v|),
    codes = E2M1(v * 2^-e). Returns (codes uint8 [..., L], scale bytes uint8 e+127)."""
    v = np.asarray(v, dtype=np.float32)
    *lead, L = v.shape
    assert L % block == 0
    g = v.reshape(*lead, L // block, block).astype(np.float64)
    e = e8m0_exponent(np.abs(g).max(axis=-1))
    scaled = g * np.exp2(-e.astype(np.float64))[..., None]
    codes = e2m1_encode(scaled)
    return codes.reshape(*lead, L), (e + 127).astype(np.uint8)


def dequant_int4(q: np.ndarray, s: np.ndarray, group: int = GROUP_INT4) -> np.ndarray:
    *lead, L = q.shape
    g = q.astype(np.float64).reshape(*lead, L // group, group)
    return (g * s.astype(np.float64)[..., None]).reshape(*lead, L)


def dequant_mxfp4(codes: np.ndarray, sbytes: np.ndarray, block: int = BLOCK_MX) -> np.ndarray:
    *lead, L = codes.shape
    vals = e2m1_decode(codes).reshape(*lead, L // block, block)
    sc = np.exp2(sbytes.astype(np.float64) - 127.0)
    return (vals * sc[..., None]).reshape(*lead, L)


# ----------------------------------------------------------------------------
# pack and forward
# ----------------------------------------------------------------------------
def pack(w_lin: np.ndarray, bias: np.ndarray, act_absmax: np.ndarray, rank: int,
         fmt: str, round_bf16: bool = True, factors=None) -> dict:
    """Offline preparation of one layer. fmt in {"int4", "mxfp4", "none"}.

    ``factors`` = (mu, l1, l2) skips steps 1-2 and uses the given smoothing and
    factors (mu float32 [K]; l1 [K][r], l2 [r][N] holding bf16 values).
    "none" keeps the residual unquantized (used by the closed-form checks).
    """
    w_lin = np.asarray(w_lin, dtype=np.float32)
    N, K = w_lin.shape
    if factors is None:
        _, mu = smoothing_factors(act_absmax, w_lin)
        w_hat = smoothed_weight(w_lin, mu)
        l1, l2 = low_rank_factors(w_hat, rank, round_bf16=round_bf16)
    else:
        mu, l1, l2 = factors
        mu = np.asarray(mu, dtype=np.float32)
        w_hat = smoothed_weight(w_lin, mu)
    r_math = residual(w_hat, l1, l2)
    out = dict(fmt=fmt, K=K, N=N, rank=rank, mu=mu, l1=l1, l2=l2,
               bias=np.zeros(N, np.float32) if bias is None else np.asarray(bias, np.float32),
               w_hat=w_hat)
    r_lin = np.ascontiguousarray(np.asarray(r_math).T)   # [N][K]
    out["r"] = r_lin
    if fmt == "int4":
        out["qw"], out["sw"] = quant_int4_rows(r_lin)
    elif fmt == "mxfp4":
        out["qw"], out["sw"] = quant_mxfp4_rows(r_lin)
    elif fmt != "none":
        raise ValueError(fmt)
    return out


def quantize_activations(x_hat: np.ndarray, fmt: str):
    if fmt == "int4":
        return quant_int4_rows(x_hat)
    if fmt == "mxfp4":
        return quant_mxfp4_rows(x_hat)
    raise ValueError(fmt)


def int4_group_sums(qx: np.ndarray, qw: np.ndarray, group: int = GROUP_INT4) -> np.ndarray:
    """P[m,n,g] = sum_{k in group g} qx[m,k] qw[n,k], exact (int32)."""
    M, K = qx.shape
    N = qw.shape[0]
    G = K // group
    P = np.empty((M, N, G), dtype=np.int32)
    for g in range(G):
        a = qx[:, g * group:(g + 1) * group].astype(np.float64)
        b = qw[:, g * group:(g + 1) * group].astype(np.float64)
        P[:, :, g] = (a @ b.T).astype(np.int32)        # |P| <= 64*49: exact in float64
    return P


def forward(packed: dict, x: np.ndarray, return_parts: bool = False):
    """Y [M][N] float64 for X [M][K] (float32 values of bf16 inputs)."""
    fmt = packed["fmt"]
    x_hat = smooth_activations(x, packed["mu"])
    l1 = np.asarray(packed["l1"], dtype=np.float64)
    l2 = np.asarray(packed["l2"], dtype=np.float64)
    z = x_hat.astype(np.float64) @ l1                            # [M][r]
    y_lr = z @ l2
    if fmt == "none":
        y_q = x_hat.astype(np.float64) @ np.asarray(packed["r"], np.float64).T
        qx = sx = None
    else:
        qx, sx = quantize_activations(x_hat, fmt)
        if fmt == "int4":
            xd = dequant_int4(qx, sx)
            wd = dequant_int4(packed["qw"], packed["sw"])
        else:
            xd = dequant_mxfp4(qx, sx)
            wd = dequant_mxfp4(packed["qw"], packed["sw"])
        y_q = xd @ wd.T
    y = y_lr + y_q + packed["bias"].astype(np.float64)[None, :]
    if return_parts:
        return y, dict(x_hat=x_hat, qx=qx, sx=sx, z=z, y_lr=y_lr, y_q=y_q)
    return y


# ----------------------------------------------------------------------------
# LoRA adapters on a packed layer, without re-quantization
# ----------------------------------------------------------------------------
def lora_extend(packed: dict, lora_a: np.ndarray, lora_b: np.ndarray, scale: float) -> dict:
    """A packed layer that also applies a LoRA adapter, with its 4-bit residual
    left as it is (aiflownews.com, "What SVDQuant actually does": pre-trained
    low-rank adapters are used without quantizing again).

    The adapter adds scale * X A B to Y (A [K][r_a], B [r_a][N], math layout).
    The layer sees X_hat = X diag(mu), so X = X_hat diag(1/mu) and the adapter
    is the low-rank product X_hat (diag(1/mu) A scale) B, which joins the
    16-bit branch: L1' = [L1 | bf16(A[k,i] * scale / mu_k)] (taken in float64,
    multiply then divide, one bf16 rounding) and L2' = [L2 ; bf16(B)]. mu, the
    residual's codes and scales and the bias are the base layer's.
    """
    a = np.asarray(lora_a, dtype=np.float32).astype(np.float64)
    b = np.asarray(lora_b, dtype=np.float32).astype(np.float64)
    K, ra = a.shape
    assert b.shape == (ra, packed["N"]) and K == packed["K"]
    mu = np.asarray(packed["mu"], dtype=np.float32).astype(np.float64)
    l1a = to_bf16((a * np.float64(np.float32(scale))) / mu[:, None])
    l2a = to_bf16(b)
    out = dict(packed)
    out["rank"] = packed["rank"] + ra
    out["l1"] = np.concatenate([np.asarray(packed["l1"], np.float32).reshape(K, -1), l1a], axis=1)
    out["l2"] = np.concatenate([np.asarray(packed["l2"], np.float32).reshape(-1, packed["N"]), l2a], axis=0)
    return out


def forward_rows(packed: dict, x_rows: np.ndarray) -> np.ndarray:
    """Forward for a subset of token rows (rows are independent in every step)."""
    return forward(packed, x_rows)


# ----------------------------------------------------------------------------
# Two layers with a GELU between (the MLP of a transformer block)
# ----------------------------------------------------------------------------
def gelu(v) -> np.ndarray:
    """GELU(v) = v Phi(v), Phi the standard normal distribution function,
    Phi(v) = erfc(-v / sqrt 2) / 2 (float64)."""
    from scipy.special import erfc
    v = np.asarray(v, dtype=np.float64)
    return v * (0.5 * erfc(-v / math.sqrt(2.0)))


def mlp_forward(up: dict, down: dict, x: np.ndarray) -> np.ndarray:
    """Y [M][N_down] float64 = down(bf16(GELU(bf16(up(X))))): each layer's
    output is rounded to bf16 as the layer writes it, and so is the GELU's."""
    h = to_bf16(gelu(to_bf16(forward(up, x))))
    return forward(down, h)

