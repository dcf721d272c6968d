"""Scalar-loop brute force for tiny shapes -- TEST INFRASTRUCTURE ONLY.

A second, deliberately naive statement of the same layer (plain Python
loops over single numbers, Python floats for float64 and numpy.float32
scalars where the method fixes float32). It shares no helper with
svdq_oracle.py; the tests require the two to agree bit for bit on codes,
scales and residuals, and to rounding on Y.

Method steps as in svdq_oracle.py (aiflownews.com page, "What SVDQuant
actually does": smoothing, SVD low-rank branch, 4-bit residual and
activations; t3chbillion.com page: W4A4).
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32


def _rne_half_even(t: float) -> int:
    """Round a float64 to the nearest integer, ties to even (by hand)."""
    fl = math.floor(t)
    frac = t - fl
    if frac > 0.5:
        return fl + 1
    if frac < 0.5:
        return fl
    return fl if fl % 2 == 0 else fl + 1


def int4_group(vals):
    """One group: returns (codes list[int], scale float32)."""
    amax = F32(0.0)
    for v in vals:
        if abs(F32(v)) > amax:
            amax = abs(F32(v))
    s = F32(amax) / F32(7.0)             # float32 / float32 -> float32 (IEEE)
    codes = []
    for v in vals:
        if s == 0:
            codes.append(0)
            continue
        q = _rne_half_even(float(F32(v)) / float(s))
        codes.append(max(-7, min(7, q)))
    return codes, F32(s)


# E2M1 magnitudes listed in code order (code bits e1 e0 m)
_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_code(v: float) -> int:
    a = abs(v)
    if a >= 6.0:
        c = 7
    else:
        best, bestd = None, None
        for code, g in enumerate(_E2M1):
            d = abs(a - g)
            if bestd is None or d < bestd or (d == bestd and (code & 1) == 0 and (best & 1) == 1):
                best, bestd = code, d
        c = best
    if math.copysign(1.0, v) < 0:
        c |= 8
    return c


def mx_block(vals):
    """One block of 32: returns (codes list[int], scale byte)."""
    amax = 0.0
    for v in vals:
        amax = max(amax, abs(float(F32(v))))
    if amax == 0.0:
        e = -127
    else:
        e = math.floor(math.log2(amax))
        # guard log2 rounding right at powers of two
        while 2.0 ** e > amax:
            e -= 1
        while 2.0 ** (e + 1) <= amax:
            e += 1
        e = max(-127, min(127, e - 2))
    codes = [e2m1_code(float(F32(v)) * 2.0 ** (-e)) for v in vals]
    return codes, e + 127


def bf16_round(v: float) -> float:
    """Nearest bf16 value of a real, ties to even (8 significant bits from
    2^-126 up; below it the subnormals, spaced 2^-133)."""
    if v == 0.0:
        return 0.0
    e = math.floor(math.log2(abs(v)))
    while 2.0 ** e > abs(v):
        e -= 1
    while 2.0 ** (e + 1) <= abs(v):
        e += 1
    ulp = 2.0 ** (max(e, -126) - 7)
    q = _rne_half_even(v / ulp)
    return q * ulp


def pack(w_lin, bias, ax, l1, l2, fmt, mu=None):
    """w_lin [N][K]; ax [K]; factors l1 [K][r], l2 [r][N] given (bf16 values).

    Returns dict with mu, codes [N][K], scales [N][K/g], residual [N][K] (float32).
    """
    N = len(w_lin)
    K = len(w_lin[0])
    r = len(l1[0]) if K and len(l1) else 0
    if mu is None:
        mu = []
        for k in range(K):
            aw = 0.0
            for n in range(N):
                aw = max(aw, abs(float(w_lin[n][k])))
            a = float(F32(ax[k]))
            lam = math.sqrt(a / aw) if (a > 0 and aw > 0) else 1.0
            mu.append(F32(1.0 / lam))
    R = [[0.0] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            what = float(F32(w_lin[n][k])) / float(mu[k])
            acc = 0.0
            for i in range(r):
                acc = acc + float(l1[k][i]) * float(l2[i][n])
            R[n][k] = F32(what - acc)
    codes = [[0] * K for _ in range(N)]
    g = 64 if fmt == "int4" else 32
    scales = [[0] * (K // g) for _ in range(N)]
    for n in range(N):
        for j in range(K // g):
            chunk = R[n][j * g:(j + 1) * g]
            if fmt == "int4":
                c, s = int4_group(chunk)
            else:
                c, s = mx_block(chunk)
            codes[n][j * g:(j + 1) * g] = c
            scales[n][j] = s
    return dict(mu=mu, R=R, codes=codes, scales=scales, fmt=fmt, l1=l1, l2=l2,
                bias=[float(b) for b in bias])


def _val(code, scale, fmt):
    if fmt == "int4":
        return float(code) * float(scale)
    mag = _E2M1[code & 7]
    return (-mag if code & 8 else mag) * 2.0 ** (int(scale) - 127)


def forward(p, x):
    """x [M][K] floats. Returns (Y [M][N] float64, codes, scales, Z)."""
    fmt = p["fmt"]
    M = len(x)
    K = len(p["mu"])
    N = len(p["codes"])
    r = len(p["l1"][0]) if len(p["l1"]) else 0
    g = 64 if fmt == "int4" else 32
    xh = [[F32(F32(x[m][k]) * p["mu"][k]) for k in range(K)] for m in range(M)]
    xc = [[0] * K for _ in range(M)]
    xs = [[0] * (K // g) for _ in range(M)]
    for m in range(M):
        for j in range(K // g):
            chunk = xh[m][j * g:(j + 1) * g]
            c, s = int4_group(chunk) if fmt == "int4" else mx_block(chunk)
            xc[m][j * g:(j + 1) * g] = c
            xs[m][j] = s
    Z = [[sum(float(xh[m][k]) * float(p["l1"][k][i]) for k in range(K)) for i in range(r)]
         for m in range(M)]
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            lr = sum(Z[m][i] * float(p["l2"][i][n]) for i in range(r))
            q = 0.0
            for k in range(K):
                q += _val(xc[m][k], xs[m][k // g], fmt) * _val(p["codes"][n][k], p["scales"][n][k // g], fmt)
            Y[m][n] = lr + q + p["bias"][n]
    return Y, xc, xs, Z


def gelu(v: float) -> float:
    """v (1 + erf(v / sqrt 2)) / 2 for one number."""
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def mlp_forward(p_up, p_down, x):
    """The down layer on bf16(GELU(bf16(up(x)))), one number at a time."""
    y_up = forward(p_up, x)[0]
    h = [[bf16_round(gelu(bf16_round(v))) for v in row] for row in y_up]
    return forward(p_down, h)[0]

