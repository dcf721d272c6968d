// Offline preparation of an SVDQuant W4A4 layer (host C++, no GPU).
//
// Steps, in the order the aiflownews.com page gives them ("What SVDQuant
// actually does"): move activation outliers into the weights (smoothing),
// split the smoothed weight by SVD into a bf16 low-rank branch and a
// residual, quantize the residual to 4 bits. The SVD is a randomized
// subspace iteration (Halko, Martinsson and Tropp, "Finding structure with
// randomness", 2011: Gaussian range finder + power iterations) followed by a
// one-sided Jacobi SVD (Hestenes) of the small projected matrix; no LAPACK.
//
// This file must be compiled without floating-point contraction
// (-ffp-contract=off) and without fast-math: the residual and the quantizer
// are defined bit for bit.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <functional>
#include <thread>
#include <vector>

#include "svdq.h"
#include "svdq_layout.h"
#include "svdq_pack_host.h"

namespace svdq {
namespace {

int n_threads() {
  unsigned h = std::thread::hardware_concurrency();
  if (h == 0) h = 1;
  return (int)std::min(h, 32u);
}

// Run fn(begin, end) over [0, n) split into contiguous chunks on worker threads.
void parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& fn) {
  int T = n_threads();
  if (n < 64 || T == 1) { fn(0, n); return; }
  T = (int)std::min<int64_t>(T, n);
  std::vector<std::thread> th;
  int64_t chunk = (n + T - 1) / T;
  for (int t = 0; t < T; ++t) {
    int64_t b = t * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    th.emplace_back(fn, b, e);
  }
  for (auto& x : th) x.join();
}

}  // namespace

// ---------------- bf16 ----------------
// Round a real to the nearest bf16 (8 significant bits), ties to even, in one
// rounding: v = f 2^e with f in [0.5, 1) -> nearbyint(f 2^8) 2^(e-8).
uint16_t bf16_from_double(double v) {
  float f32;
  if (v == 0.0 || !std::isfinite(v)) {
    f32 = (float)v;
  } else {
    int e;
    double f = std::frexp(v, &e);
    double m = std::nearbyint(f * 256.0);
    f32 = (float)std::ldexp(m, e - 8);   // exact: 8-bit significand
  }
  uint32_t u;
  std::memcpy(&u, &f32, 4);
  return (uint16_t)(u >> 16);
}
double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

namespace {

// ---------------- seeded Gaussian (splitmix64 + Box-Muller) ----------------
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
  double normal() {
    double u1 = uniform(), u2 = uniform();
    return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
  }
};

// ---------------- dense helpers (row-major, fp64) ----------------
// Y[K][L] = A[K][N] * X[N][L]
void mul_AX(const double* A, int64_t K, int64_t N, const double* X, int L, double* Y) {
  parallel_for(K, [&](int64_t b, int64_t e) {
    std::vector<double> acc(L);
    for (int64_t k = b; k < e; ++k) {
      std::fill(acc.begin(), acc.end(), 0.0);
      const double* a = A + k * N;
      for (int64_t n = 0; n < N; ++n) {
        double av = a[n];
        const double* x = X + n * L;
        for (int j = 0; j < L; ++j) acc[j] += av * x[j];
      }
      std::copy(acc.begin(), acc.end(), Y + k * L);
    }
  });
}
// Y[N][L] = A^T * X, A[K][N], X[K][L]
void mul_AtX(const double* A, int64_t K, int64_t N, const double* X, int L, double* Y) {
  parallel_for(N, [&](int64_t b, int64_t e) {
    int64_t w = e - b;
    std::vector<double> acc((size_t)w * L, 0.0);
    for (int64_t k = 0; k < K; ++k) {
      const double* a = A + k * N + b;
      const double* x = X + k * L;
      for (int64_t n = 0; n < w; ++n) {
        double av = a[n];
        double* o = acc.data() + n * L;
        for (int j = 0; j < L; ++j) o[j] += av * x[j];
      }
    }
    std::copy(acc.begin(), acc.end(), Y + b * L);
  });
}

// Orthonormalize the L columns of Q[R][L] in place (Gram-Schmidt run twice).
// Columns that vanish are replaced by zeros (rank-deficient input).
void orthonormalize(double* Q, int64_t R, int L) {
  std::vector<double> dots(L);
  for (int j = 0; j < L; ++j) {
    for (int pass = 0; pass < 2; ++pass) {
      std::fill(dots.begin(), dots.end(), 0.0);
      for (int64_t i = 0; i < R; ++i) {
        const double* row = Q + i * L;
        for (int p = 0; p < j; ++p) dots[p] += row[p] * row[j];
      }
      for (int64_t i = 0; i < R; ++i) {
        double* row = Q + i * L;
        double v = row[j];
        for (int p = 0; p < j; ++p) v -= dots[p] * row[p];
        row[j] = v;
      }
    }
    double nrm = 0.0;
    for (int64_t i = 0; i < R; ++i) nrm += Q[i * L + j] * Q[i * L + j];
    nrm = std::sqrt(nrm);
    double inv = nrm > 1e-300 ? 1.0 / nrm : 0.0;
    for (int64_t i = 0; i < R; ++i) Q[i * L + j] *= inv;
  }
}

// One-sided Jacobi SVD of A [R][L] (columns rotated until mutually
// orthogonal). On return A's columns are V_j sigma_j and J [L][L] holds the
// accumulated rotations, so that A_in = A_out J^T. Returns false if not
// converged within the sweep cap.
bool one_sided_jacobi(double* A, int64_t R, int L, double* J, int max_sweeps) {
  for (int i = 0; i < L; ++i)
    for (int j = 0; j < L; ++j) J[i * L + j] = (i == j) ? 1.0 : 0.0;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < L - 1; ++p) {
      for (int q = p + 1; q < L; ++q) {
        double alpha = 0, beta = 0, gamma = 0;
        for (int64_t i = 0; i < R; ++i) {
          double ap = A[i * L + p], aq = A[i * L + q];
          alpha += ap * ap;
          beta += aq * aq;
          gamma += ap * aq;
        }
        if (alpha == 0.0 || beta == 0.0) continue;
        double c_ = std::fabs(gamma) / std::sqrt(alpha * beta);
        off = std::max(off, c_);
        if (c_ < 1e-15) continue;
        double zeta = (beta - alpha) / (2.0 * gamma);
        double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int64_t i = 0; i < R; ++i) {
          double ap = A[i * L + p], aq = A[i * L + q];
          A[i * L + p] = c * ap - s * aq;
          A[i * L + q] = s * ap + c * aq;
        }
        for (int i = 0; i < L; ++i) {
          double jp = J[i * L + p], jq = J[i * L + q];
          J[i * L + p] = c * jp - s * jq;
          J[i * L + q] = s * jp + c * jq;
        }
      }
    }
    if (off < 1e-12) return true;
  }
  return false;
}

int jacobi_sweeps();

}  // namespace

// Top-r factors of the K x N matrix W_hat that AX (W_hat X, X [N][L] -> [K][L])
// and AtX (W_hat^T X, X [K][L] -> [N][L]) apply: L1 [K][r] = U_r Sigma_r,
// L2 [r][N] = V_r^T (fp64), by randomized subspace iteration (Halko,
// Martinsson and Tropp) with the small factorizations on the host.
svdq_status truncated_svd_ops(int64_t K, int64_t N, int r, uint64_t seed, const PanelOp& AX, const PanelOp& AtX,
                              std::vector<double>& L1, std::vector<double>& L2) {
  // oversampled subspace; power iterations until the captured energy
  // ||W Z||_F^2 stops growing (relative change below 1e-9), at most 60
  const int L = (int)std::min<int64_t>(r + std::max(16, r / 2), std::min(K, N));
  const int max_power_iters = 60;
  Rng rng{seed ^ 0x5EED5EED12345678ull};
  std::vector<double> Om((size_t)N * L), Y((size_t)K * L), Z((size_t)N * L);
  for (auto& v : Om) v = rng.normal();
  svdq_status st = AX(Om.data(), Y.data());
  if (st != SVDQ_OK) return st;
  orthonormalize(Y.data(), K, L);
  double prev = -1.0;
  for (int it = 0; it < max_power_iters; ++it) {
    if ((st = AtX(Y.data(), Z.data())) != SVDQ_OK) return st;
    orthonormalize(Z.data(), N, L);
    if ((st = AX(Z.data(), Y.data())) != SVDQ_OK) return st;
    double energy = 0.0;
    for (size_t i = 0; i < Y.size(); ++i) energy += Y[i] * Y[i];
    orthonormalize(Y.data(), K, L);
    if (!std::isfinite(energy)) return SVDQ_ERR_NUMERIC;
    if (prev > 0 && energy - prev <= 1e-9 * energy) break;
    prev = energy;
  }
  // B^T = W^T Q  [N][L]; B = Q^T W
  if ((st = AtX(Y.data(), Z.data())) != SVDQ_OK) return st;
  std::vector<double> J((size_t)L * L);
  if (!one_sided_jacobi(Z.data(), N, L, J.data(), jacobi_sweeps())) return SVDQ_ERR_NUMERIC;
  // B^T = (V Sigma) J^T  ->  B = J Sigma V^T, W ~= Q B = (Q J) Sigma V^T
  std::vector<double> sig(L);
  for (int j = 0; j < L; ++j) {
    double s = 0;
    for (int64_t i = 0; i < N; ++i) s += Z[i * L + j] * Z[i * L + j];
    sig[j] = std::sqrt(s);
  }
  std::vector<int> order(L);
  for (int j = 0; j < L; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return sig[a] > sig[b]; });
  L1.assign((size_t)K * r, 0.0);
  L2.assign((size_t)r * N, 0.0);
  for (int c = 0; c < r; ++c) {
    int j = order[c];
    double s = sig[j];
    if (!std::isfinite(s)) return SVDQ_ERR_NUMERIC;
    // L1[:, c] = Q J[:, j] sigma_j ; L2[c, :] = V_j^T = Z[:, j]^T / sigma_j
    for (int64_t k = 0; k < K; ++k) {
      double acc = 0;
      for (int p = 0; p < L; ++p) acc += Y[k * L + p] * J[p * L + j];
      L1[k * r + c] = acc * s;
    }
    double inv = s > 0 ? 1.0 / s : 0.0;
    for (int64_t n = 0; n < N; ++n) L2[c * N + n] = Z[n * L + j] * inv;
  }
  return SVDQ_OK;
}

svdq_status smoothing_mu(int K, const float* ax, const float* aw, double alpha, float* mu) {
  for (int k = 0; k < K; ++k) {
    const double a = (double)ax[k], w = (double)aw[k];
    double lam = 1.0;
    if (a > 0 && w > 0) lam = alpha == 0.5 ? std::sqrt(a / w) : std::pow(a, alpha) / std::pow(w, 1.0 - alpha);
    mu[k] = (float)(1.0 / lam);
    if (!(mu[k] > 0.f) || !std::isfinite(mu[k])) return SVDQ_ERR_NUMERIC;
  }
  return SVDQ_OK;
}

void factor_layout(const svdq_layer_desc* d, const uint16_t* l1b, const uint16_t* l2b, uint16_t* l1_out,
                   uint16_t* l2_out) {
  const int K = d->K, N = d->N, r = d->rank, r32 = rank32(r), Kp = kpad(d);
  const svdq_packed_sizes sz = packed_sizes(d);
  std::memset(l1_out, 0, sz.l1);
  std::memset(l2_out, 0, sz.l2);
  for (int k = 0; k < K; ++k)
    for (int c = 0; c < r; ++c) l1_out[l1_index(Kp, r32, k, c)] = l1b[(size_t)k * r + c];
  for (int i = 0; i < r; ++i)
    for (int n = 0; n < N; ++n) l2_out[frag16_index(r32, n, i)] = l2b[(size_t)i * N + n];
}

namespace {

// Top-r factors of W_hat [K][N] in host memory.
svdq_status truncated_svd(const double* W, int64_t K, int64_t N, int r, uint64_t seed,
                          std::vector<double>& L1, std::vector<double>& L2) {
  const int L = (int)std::min<int64_t>(r + std::max(16, r / 2), std::min(K, N));
  return truncated_svd_ops(
      K, N, r, seed,
      [&](const double* X, double* Y) {
        mul_AX(W, K, N, X, L, Y);
        return SVDQ_OK;
      },
      [&](const double* X, double* Y) {
        mul_AtX(W, K, N, X, L, Y);
        return SVDQ_OK;
      },
      L1, L2);
}

// ---------------- 4-bit quantizers (definitions as in svdq.h) ----------------
// INT4: s = fl32(amax / 7); q = round-half-to-even(v / s) of the exact
// quotient (the fp64 quotient of two fp32 values decides every half-integer
// correctly), clamped to [-7, 7]; amax == 0 -> s = 0, q = 0.
void quant_int4_group(const float* v, int n, int8_t* q, float* s_out) {
  float amax = 0.f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  float s = amax / 7.0f;
  *s_out = s;
  for (int i = 0; i < n; ++i) {
    if (s == 0.f) { q[i] = 0; continue; }
    double t = std::nearbyint((double)v[i] / (double)s);
    t = std::min(7.0, std::max(-7.0, t));
    q[i] = (int8_t)t;
  }
}

// E2M1 code of a real value, ties to the even mantissa bit, saturating at 6.
// Decision points are the midpoints between neighbouring E2M1 values.
uint8_t e2m1_code(double v) {
  double a = std::fabs(v);
  uint8_t c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  if (std::signbit(v)) c |= 8;
  return c;
}

// MXFP4 block: e = floor(log2 amax) - 2 clamped to [-127, 127] (amax == 0 -> -127).
void quant_mx_block(const float* v, int n, uint8_t* codes, uint8_t* sbyte) {
  float amax = 0.f;
  for (int i = 0; i < n; ++i) amax = std::max(amax, std::fabs(v[i]));
  int e = -127;
  if (amax > 0.f) {
    int E;
    std::frexp((double)amax, &E);   // amax = f 2^E, f in [0.5, 1)
    e = std::max(-127, std::min(127, (E - 1) - 2));
  }
  *sbyte = (uint8_t)(e + 127);
  for (int i = 0; i < n; ++i) codes[i] = e2m1_code(std::ldexp((double)v[i], -e));
}

bool all_finite(const float* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

bool packed_ok(const svdq_packed* p) { return p && p->mu && p->qw && p->sw && p->bias; }

// Sweep cap of the Jacobi step; SVDQ_JACOBI_MAX_SWEEPS overrides it (used by
// the tests to force the non-convergence error path from the host).
int jacobi_sweeps() {
  const char* e = std::getenv("SVDQ_JACOBI_MAX_SWEEPS");
  if (e && *e) return std::max(0, std::atoi(e));
  return 60;
}

// Residual (fp64, increasing rank index, no contraction), quantization and
// device layout of the weight side. l1b [K][r], l2b [r][N] are bf16 bits.
svdq_status finish_pack(const svdq_layer_desc* d, const float* w_lin, const float* bias,
                        const float* mu, const uint16_t* l1b, const uint16_t* l2b,
                        svdq_packed* out) {
  const int K = d->K, N = d->N, r = d->rank, r32 = rank32(r);
  const int Kp = kpad(d), Np = npad(d);
  if (r32 > 0 && (!out->l1 || !out->l2)) return SVDQ_ERR_NULL;
  const svdq_packed_sizes sz = packed_sizes(d);
  std::memcpy(out->mu, mu, (size_t)K * 4);
  // the padding (channels K..Kp, rows N..Np) stays zero
  std::memset(out->qw, 0, sz.qw);
  std::memset(out->sw, 0, sz.sw);
  std::memset(out->bias, 0, sz.bias);
  // factors in device layout
  if (r32 > 0) factor_layout(d, l1b, l2b, out->l1, out->l2);
  for (int n = 0; n < N; ++n) {
    float b = bias ? bias[n] : 0.f;
    out->bias[n] = bf16_from_double((double)b);
  }
  std::vector<double> l1d((size_t)K * r), l2d((size_t)r * N);
  for (size_t i = 0; i < l1d.size(); ++i) l1d[i] = bf16_to_double(l1b[i]);
  for (size_t i = 0; i < l2d.size(); ++i) l2d[i] = bf16_to_double(l2b[i]);
  const int G = d->format == SVDQ_FMT_INT4_G64 ? K / kGroupInt4 : K / kBlockMx;
  const int gsz = d->format == SVDQ_FMT_INT4_G64 ? kGroupInt4 : kBlockMx;
  float* sw_f = (float*)out->sw;
  uint8_t* sw_b = (uint8_t*)out->sw;
  parallel_for(N, [&](int64_t b, int64_t e) {
    std::vector<float> rrow(K);
    std::vector<int8_t> q(gsz);
    std::vector<uint8_t> cq(gsz);
    for (int64_t n = b; n < e; ++n) {
      for (int k = 0; k < K; ++k) {
        double what = (double)w_lin[(size_t)n * K + k] / (double)mu[k];
        double acc = 0.0;
        for (int i = 0; i < r; ++i) {
          double prod = l1d[(size_t)k * r + i] * l2d[(size_t)i * N + n];
          acc = acc + prod;
        }
        rrow[k] = (float)(what - acc);
      }
      for (int g = 0; g < G; ++g) {
        if (d->format == SVDQ_FMT_INT4_G64) {
          float s;
          quant_int4_group(&rrow[(size_t)g * gsz], gsz, q.data(), &s);
          sw_f[(size_t)g * Np + n] = s;
          for (int j = 0; j < gsz; j += 2)
            out->qw[f_code_byte(Kp, n, g * gsz + j)] = (uint8_t)((q[j] & 15) | ((q[j + 1] & 15) << 4));
        } else {
          uint8_t sb;
          quant_mx_block(&rrow[(size_t)g * gsz], gsz, cq.data(), &sb);
          sw_b[f_scale_index(Np, n, g)] = sb;
          for (int j = 0; j < gsz; j += 2)
            out->qw[f_code_byte(Kp, n, g * gsz + j)] = (uint8_t)((cq[j] & 15) | ((cq[j + 1] & 15) << 4));
        }
      }
    }
  });
  return SVDQ_OK;
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

const char* svdq_status_string(svdq_status s) {
  switch (s) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_ERR_NULL: return "SVDQ_ERR_NULL: a required pointer is NULL";
    case SVDQ_ERR_SHAPE: return "SVDQ_ERR_SHAPE: unsupported K/N/rank/M or window";
    case SVDQ_ERR_FORMAT: return "SVDQ_ERR_FORMAT: unknown format";
    case SVDQ_ERR_WORKSPACE: return "SVDQ_ERR_WORKSPACE: workspace too small";
    case SVDQ_ERR_NUMERIC: return "SVDQ_ERR_NUMERIC: non-finite input or SVD did not converge";
    case SVDQ_ERR_DEVICE: return "SVDQ_ERR_DEVICE: not a gfx950 device, or a HIP call failed";
  }
  return "SVDQ_ERR_UNKNOWN";
}

int32_t svdq_version(void) { return 100; }

svdq_status svdq_packed_bytes(const svdq_layer_desc* d, svdq_packed_sizes* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  *out = packed_sizes(d);
  return SVDQ_OK;
}

svdq_status svdq_workspace_bytes(const svdq_layer_desc* d, int64_t M, size_t* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  *out = ws_layout(d, M).total;
  return SVDQ_OK;
}

svdq_status svdq_quantize_residual(const svdq_layer_desc* d, const float* w_lin, const float* bias,
                                   const float* mu, const uint16_t* l1, const uint16_t* l2,
                                   svdq_packed* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!w_lin || !mu || !packed_ok(out)) return SVDQ_ERR_NULL;
  if (d->rank > 0 && (!l1 || !l2)) return SVDQ_ERR_NULL;
  const size_t K = d->K, N = d->N;
  if (!all_finite(w_lin, N * K) || !all_finite(mu, K) || (bias && !all_finite(bias, N)))
    return SVDQ_ERR_NUMERIC;
  for (size_t k = 0; k < K; ++k)
    if (!(mu[k] > 0.f)) return SVDQ_ERR_NUMERIC;
  return finish_pack(d, w_lin, bias, mu, l1, l2, out);
}

svdq_status svdq_pack_weights(const svdq_layer_desc* d, const float* w_lin, const float* bias,
                              const float* act_absmax, uint64_t seed, svdq_packed* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!w_lin || !act_absmax || !packed_ok(out)) return SVDQ_ERR_NULL;
  const int64_t K = d->K, N = d->N;
  const int r = d->rank;
  if (!all_finite(w_lin, (size_t)N * K) || !all_finite(act_absmax, K) ||
      (bias && !all_finite(bias, N)))
    return SVDQ_ERR_NUMERIC;
  // 1. smoothing: lambda_k = sqrt(max|X_k| / max|W_k|), mu_k = fl32(1 / lambda_k)
  std::vector<float> aw(K, 0.f), mu(K);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) aw[k] = std::max(aw[k], std::fabs(w_lin[n * K + k]));
  st = smoothing_mu((int)K, act_absmax, aw.data(), 0.5, mu.data());
  if (st != SVDQ_OK) return st;
  // 2. low-rank branch of W_hat = diag(1/mu) W  (math layout [K][N], fp64)
  std::vector<uint16_t> l1b((size_t)K * r), l2b((size_t)r * N);
  if (r > 0) {
    std::vector<double> W((size_t)K * N);
    parallel_for(K, [&](int64_t b, int64_t e) {
      for (int64_t k = b; k < e; ++k)
        for (int64_t n = 0; n < N; ++n)
          W[k * N + n] = (double)w_lin[n * K + k] / (double)mu[k];
    });
    std::vector<double> L1, L2;
    st = truncated_svd(W.data(), K, N, r, seed, L1, L2);
    if (st != SVDQ_OK) return st;
    for (size_t i = 0; i < L1.size(); ++i) l1b[i] = bf16_from_double(L1[i]);
    for (size_t i = 0; i < L2.size(); ++i) l2b[i] = bf16_from_double(L2[i]);
  }
  // 3. residual against the bf16 factors, 4-bit quantization, device layout
  return finish_pack(d, w_lin, bias, mu.data(), l1b.data(), l2b.data(), out);
}

svdq_status svdq_unpack_weights(const svdq_layer_desc* d, const svdq_packed* h, int8_t* codes,
                                void* scales, uint16_t* l1, uint16_t* l2, uint16_t* bias) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!h) return SVDQ_ERR_NULL;
  const int K = d->K, N = d->N, r = d->rank, r32 = rank32(r);
  const int Kp = kpad(d), Np = npad(d);
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  if (codes) {
    if (!h->qw) return SVDQ_ERR_NULL;
    for (size_t n = 0; n < (size_t)N; ++n)
      for (int k = 0; k < K; ++k) {
        uint8_t byte = h->qw[f_code_byte(Kp, n, k)];
        int nib = (k & 1) ? (byte >> 4) : (byte & 15);
        codes[n * K + k] = int4 ? (int8_t)(nib >= 8 ? nib - 16 : nib) : (int8_t)nib;
      }
  }
  if (scales) {
    if (!h->sw) return SVDQ_ERR_NULL;
    if (int4) {
      const int G = K / kGroupInt4;
      for (int n = 0; n < N; ++n)
        for (int g = 0; g < G; ++g)
          ((float*)scales)[(size_t)n * G + g] = ((const float*)h->sw)[(size_t)g * Np + n];
    } else {
      const int G = K / kBlockMx;
      for (int n = 0; n < N; ++n)
        for (int g = 0; g < G; ++g)
          ((uint8_t*)scales)[(size_t)n * G + g] = ((const uint8_t*)h->sw)[f_scale_index(Np, n, g)];
    }
  }
  if (l1 && r > 0) {
    if (!h->l1) return SVDQ_ERR_NULL;
    for (int k = 0; k < K; ++k)
      for (int c = 0; c < r; ++c) l1[(size_t)k * r + c] = h->l1[l1_index(Kp, r32, k, c)];
  }
  if (l2 && r > 0) {
    if (!h->l2) return SVDQ_ERR_NULL;
    for (int i = 0; i < r; ++i)
      for (int n = 0; n < N; ++n)
        l2[(size_t)i * N + n] = h->l2[frag16_index(r32, n, i)];
  }
  if (bias) {
    if (!h->bias) return SVDQ_ERR_NULL;
    std::memcpy(bias, h->bias, (size_t)N * 2);
  }
  return SVDQ_OK;
}

svdq_status svdq_lora_extend(const svdq_layer_desc* base, const svdq_packed* h, int32_t lora_rank,
                             const float* lora_a, const float* lora_b, float scale, svdq_packed* out) {
  svdq_status st = check_desc(base);
  if (st != SVDQ_OK) return st;
  if (!h || !out || !lora_a || !lora_b || !h->mu) return SVDQ_ERR_NULL;
  if (lora_rank <= 0) return SVDQ_ERR_SHAPE;
  svdq_layer_desc ed = *base;
  ed.rank = base->rank + lora_rank;
  st = check_desc(&ed);
  if (st != SVDQ_OK) return st;
  if (!out->l1 || !out->l2 || (base->rank > 0 && (!h->l1 || !h->l2))) return SVDQ_ERR_NULL;
  const int K = base->K, N = base->N, r0 = base->rank, r = ed.rank, r32 = rank32(r);
  const int r032 = rank32(r0), Kp = kpad(base);
  if (!all_finite(lora_a, (size_t)K * lora_rank) || !all_finite(lora_b, (size_t)lora_rank * N) ||
      !std::isfinite(scale))
    return SVDQ_ERR_NUMERIC;
  for (int k = 0; k < K; ++k)
    if (!(h->mu[k] > 0.f) || !std::isfinite(h->mu[k])) return SVDQ_ERR_NUMERIC;
  // the base factors (logical), then the adapter's columns of L1 and rows of L2
  std::vector<uint16_t> l1((size_t)K * r), l2((size_t)r * N);
  for (int k = 0; k < K; ++k) {
    for (int c = 0; c < r0; ++c) l1[(size_t)k * r + c] = h->l1[l1_index(Kp, r032, k, c)];
    for (int c = 0; c < lora_rank; ++c)
      l1[(size_t)k * r + r0 + c] =
          bf16_from_double(((double)lora_a[(size_t)k * lora_rank + c] * (double)scale) / (double)h->mu[k]);
  }
  for (int i = 0; i < r0; ++i)
    for (int n = 0; n < N; ++n) l2[(size_t)i * N + n] = h->l2[frag16_index(r032, n, i)];
  for (int i = 0; i < lora_rank; ++i)
    for (int n = 0; n < N; ++n) l2[(size_t)(r0 + i) * N + n] = bf16_from_double((double)lora_b[(size_t)i * N + n]);
  // device layout of the extended factors; the 4-bit side is copied as it is
  const svdq_packed_sizes esz = packed_sizes(&ed);
  std::memset(out->l1, 0, esz.l1);
  std::memset(out->l2, 0, esz.l2);
  for (int k = 0; k < K; ++k)
    for (int c = 0; c < r; ++c) out->l1[l1_index(Kp, r32, k, c)] = l1[(size_t)k * r + c];
  for (int i = 0; i < r; ++i)
    for (int n = 0; n < N; ++n) out->l2[frag16_index(r32, n, i)] = l2[(size_t)i * N + n];
  const svdq_packed_sizes sz = packed_sizes(base);
  if (out->mu && out->mu != h->mu) std::memcpy(out->mu, h->mu, sz.mu);
  if (out->qw && out->qw != h->qw) {
    if (!h->qw) return SVDQ_ERR_NULL;
    std::memcpy(out->qw, h->qw, sz.qw);
  }
  if (out->sw && out->sw != h->sw) {
    if (!h->sw) return SVDQ_ERR_NULL;
    std::memcpy(out->sw, h->sw, sz.sw);
  }
  if (out->bias && out->bias != h->bias) {
    if (!h->bias) return SVDQ_ERR_NULL;
    std::memcpy(out->bias, h->bias, sz.bias);
  }
  return SVDQ_OK;
}

svdq_status svdq_unpack_workspace(const svdq_layer_desc* d, int64_t M, const void* ws,
                                  size_t ws_bytes, int8_t* codes, void* scales, float* z) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!ws) return SVDQ_ERR_NULL;
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  WsLayout L = ws_layout(d, M);
  if (ws_bytes < L.total) return SVDQ_ERR_WORKSPACE;
  const uint8_t* base = (const uint8_t*)ws;
  const int K = d->K, Kp = kpad(d), r = d->rank, r32 = rank32(r);
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  if (codes) {
    const uint8_t* q = base + L.qx;
    for (int64_t m = 0; m < M; ++m)
      for (int k = 0; k < K; ++k) {
        uint8_t byte = q[f_code_byte(Kp, m, k)];
        int nib = (k & 1) ? (byte >> 4) : (byte & 15);
        codes[(size_t)m * K + k] = int4 ? (int8_t)(nib >= 8 ? nib - 16 : nib) : (int8_t)nib;
      }
  }
  if (scales) {
    if (int4) {
      const float* s = (const float*)(base + L.sx);
      const int G = K / kGroupInt4;
      const int64_t Mp = act_rows(M);
      for (int64_t m = 0; m < M; ++m)
        for (int g = 0; g < G; ++g) ((float*)scales)[(size_t)m * G + g] = s[(size_t)g * Mp + m];
    } else {
      const uint8_t* s = base + L.sx;
      const int G = K / kBlockMx;
      for (int64_t m = 0; m < M; ++m)
        for (int g = 0; g < G; ++g)
          ((uint8_t*)scales)[(size_t)m * G + g] = s[f_scale_index(round32(M), m, g)];
    }
  }
  if (z && r > 0) {
    const uint16_t* zb = (const uint16_t*)(base + L.z);
    for (int64_t m = 0; m < M; ++m)
      for (int i = 0; i < r; ++i)
        z[(size_t)m * r + i] =
            (float)bf16_to_double(zb[frag16_index(r32, m, i)]);
  }
  return SVDQ_OK;
}

}  // extern "C"
