// Host side of the AWQ-style W4A16 linear (aiflownews.com, "How Nunchaku
// four bit quantization actually works": the adaptive-normalization and
// modulation layers keep 16-bit activations and 4-bit weights, quantized the
// activation-aware way). Offline preparation, logical views and sizes; no GPU
// code here.
//
// Pack, for calibration activations X_cal [M_cal][K]:
//   a_k = mean_m |X_cal[m,k]| (float64, rows added in order);
//   for alpha on the grid 0, 1/20, ..., 19/20 (or the given alpha):
//     s_k = max(a_k, 1e-4)^alpha / sqrt(max s * min s);
//     W' = fl32(W[n,k] s_k), quantized per output channel per group of 128
//     input channels to asymmetric 4-bit codes (float32 steps):
//       scale = max(max - min, 1e-5) / 15, zero = clamp(-rint(min / scale), 0, 15),
//       q = clamp(rint(w / scale) + zero, 0, 15);
//     loss = sum over X_cal of (X diag(fl32(1/s)) dequant(W')^T - X W^T)^2;
//   the first alpha of least loss is kept. The runtime multiplies X by the
//   stored inv_s = fl32(1/s).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

#include "svdq.h"

namespace {

constexpr int kAwqGroup = 128;
constexpr int kAwqGrid = 20;

int threads() {
  unsigned h = std::thread::hardware_concurrency();
  return h == 0 ? 4 : (int)(h > 32 ? 32 : h);
}

void par_for(int64_t n, const std::function<void(int64_t, int64_t)>& fn) {
  const int T = (int)std::min<int64_t>(threads(), n);
  if (T <= 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < T; ++t) th.emplace_back(fn, n * t / T, n * (t + 1) / T);
  for (auto& x : th) x.join();
}

bool finite(const float* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

svdq_status check(const svdq_awq_desc* d) {
  if (!d) return SVDQ_ERR_NULL;
  if (d->K <= 0 || d->N <= 0 || d->K % kAwqGroup != 0 || d->K > 4096 || d->N % 16 != 0 || d->N > 65536)
    return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

// One row of W' quantized: codes [K], scales and zeros [K/128].
void quant_row(const float* w, int K, uint8_t* q, float* sc, uint8_t* z) {
  for (int g = 0; g < K / kAwqGroup; ++g) {
    const float* v = w + (size_t)g * kAwqGroup;
    float mx = v[0], mn = v[0];
    for (int j = 1; j < kAwqGroup; ++j) {
      mx = std::max(mx, v[j]);
      mn = std::min(mn, v[j]);
    }
    const float s = std::max(mx - mn, 1e-5f) / 15.0f;
    const float zf = std::min(15.0f, std::max(0.0f, -std::nearbyint(mn / s)));
    for (int j = 0; j < kAwqGroup; ++j) {
      const float t = std::nearbyint(v[j] / s) + zf;
      q[(size_t)g * kAwqGroup + j] = (uint8_t)std::min(15.0f, std::max(0.0f, t));
    }
    sc[g] = s;
    z[g] = (uint8_t)zf;
  }
}

// Device layout of the codes: [N/16][K/128][64 lanes][16 bytes]; lane
// l = 16 c + r holds row 16 nb + r, and its 4-byte word t the channels
// 128 g + 32 t + 8 c + (0..7), element 2 i in bits 4 i .. 4 i + 3 and element
// 2 i + 1 in bits 16 + 4 i .. 16 + 4 i + 3 (i = 0..3), so that
// ((w >> 4 i) & 0x000F000F) | 0x43004300 is the bf16 pair (128 + q_2i,
// 128 + q_2i+1). Scales fp32 and zero points u8: [N/16][K/128][16].
size_t code_byte(int K, int n, int k, int* shift) {
  const int nb = n / 16, r = n % 16, g = k / 128, t = (k % 128) / 32, c = (k % 32) / 8, j = k % 8;
  const int lane = 16 * c + r;
  *shift = (j & 1) * 16 + (j >> 1) * 4;
  return (((size_t)nb * (K / 128) + g) * 64 + lane) * 16 + 4 * t + (*shift >> 3);
}

}  // namespace

extern "C" {

svdq_status svdq_awq_packed_bytes(const svdq_awq_desc* d, svdq_awq_sizes* out) {
  svdq_status st = check(d);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  const size_t K = d->K, N = d->N, G = K / kAwqGroup;
  out->inv_s = K * 4;
  out->qw = N * K / 2;
  out->scales = N * G * 4;
  out->zeros = N * G;
  out->bias = N * 2;
  return SVDQ_OK;
}

svdq_status svdq_awq_pack(const svdq_awq_desc* d, const float* w_lin, const float* bias, const float* x_cal,
                          int64_t m_cal, float alpha, double* alpha_out, double* s_out, svdq_awq_packed* out) {
  svdq_status st = check(d);
  if (st != SVDQ_OK) return st;
  if (!w_lin || !x_cal || !out || !out->inv_s || !out->qw || !out->scales || !out->zeros || !out->bias)
    return SVDQ_ERR_NULL;
  if (m_cal <= 0) return SVDQ_ERR_SHAPE;
  const int K = d->K, N = d->N, G = K / kAwqGroup;
  if (!finite(w_lin, (size_t)N * K) || !finite(x_cal, (size_t)m_cal * K) || (bias && !finite(bias, N)))
    return SVDQ_ERR_NUMERIC;
  if (alpha >= 0.f && !(alpha <= 1.f)) return SVDQ_ERR_SHAPE;
  std::vector<double> a(K, 0.0);
  for (int64_t m = 0; m < m_cal; ++m)
    for (int k = 0; k < K; ++k) a[k] = a[k] + std::fabs((double)x_cal[m * K + k]);
  for (int k = 0; k < K; ++k) a[k] = a[k] / (double)m_cal;

  std::vector<double> s(K);
  std::vector<float> inv(K), ws((size_t)N * K), sc((size_t)N * G);
  std::vector<uint8_t> q((size_t)N * K), z((size_t)N * G);
  auto make = [&](double al) {
    double smax = 0.0, smin = INFINITY;
    for (int k = 0; k < K; ++k) {
      s[k] = std::pow(std::max(a[k], 1e-4), al);
      smax = std::max(smax, s[k]);
      smin = std::min(smin, s[k]);
    }
    const double norm = std::sqrt(smax * smin);
    for (int k = 0; k < K; ++k) {
      s[k] = s[k] / norm;
      inv[k] = (float)(1.0 / s[k]);
    }
    par_for(N, [&](int64_t b, int64_t e) {
      for (int64_t n = b; n < e; ++n) {
        for (int k = 0; k < K; ++k) ws[n * K + k] = (float)((double)w_lin[n * K + k] * s[k]);
        quant_row(&ws[n * K], K, &q[n * K], &sc[n * G], &z[n * G]);
      }
    });
  };
  auto loss = [&]() {
    // sum over calibration rows and outputs of (x_hat . deq_n - x . w_n)^2,
    // as x . (deq_n diag(inv_s) - w_n) in float64 with eight partial sums
    std::vector<double> part(N, 0.0);
    par_for(N, [&](int64_t b, int64_t e) {
      std::vector<double> dn(K);
      for (int64_t n = b; n < e; ++n) {
        for (int k = 0; k < K; ++k) {
          const float deq = sc[n * G + k / kAwqGroup] * ((float)q[n * K + k] - (float)z[n * G + k / kAwqGroup]);
          dn[k] = (double)deq * (double)inv[k] - (double)w_lin[n * K + k];
        }
        double tot = 0.0;
        for (int64_t m = 0; m < m_cal; ++m) {
          const float* xr = x_cal + m * K;
          double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
          for (int k = 0; k < K; k += 8)
            for (int u = 0; u < 8; ++u) acc[u] += (double)xr[k + u] * dn[k + u];
          const double e2 = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
          tot += e2 * e2;
        }
        part[n] = tot;
      }
    });
    double t = 0.0;
    for (int n = 0; n < N; ++n) t += part[n];
    return t;
  };
  double best = alpha;
  if (alpha < 0.f) {
    double bl = INFINITY;
    for (int i = 0; i < kAwqGrid; ++i) {
      make(i / (double)kAwqGrid);
      const double l = loss();
      if (!(l >= bl)) {   // the first least loss (a NaN loss never wins)
        bl = l;
        best = i / (double)kAwqGrid;
      }
    }
    if (!std::isfinite(bl)) return SVDQ_ERR_NUMERIC;
  }
  make(best);
  if (alpha_out) *alpha_out = best;
  if (s_out) std::memcpy(s_out, s.data(), (size_t)K * 8);
  std::memcpy(out->inv_s, inv.data(), (size_t)K * 4);
  std::memset(out->qw, 0, (size_t)N * K / 2);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) {
      int sh = 0;
      const size_t byte = code_byte(K, n, k, &sh);
      out->qw[byte] |= (uint8_t)(q[(size_t)n * K + k] << (sh & 7));
    }
  for (int n = 0; n < N; ++n)
    for (int g = 0; g < G; ++g) {
      const size_t i = ((size_t)(n / 16) * G + g) * 16 + n % 16;
      out->scales[i] = sc[(size_t)n * G + g];
      out->zeros[i] = z[(size_t)n * G + g];
    }
  for (int n = 0; n < N; ++n) {
    const float b = bias ? bias[n] : 0.f;
    uint32_t u;
    std::memcpy(&u, &b, 4);
    out->bias[n] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);   // bf16, nearest even
  }
  return SVDQ_OK;
}

svdq_status svdq_awq_unpack(const svdq_awq_desc* d, const svdq_awq_packed* h, uint8_t* codes, float* scales,
                            uint8_t* zeros) {
  svdq_status st = check(d);
  if (st != SVDQ_OK) return st;
  if (!h) return SVDQ_ERR_NULL;
  const int K = d->K, N = d->N, G = K / kAwqGroup;
  if (codes) {
    if (!h->qw) return SVDQ_ERR_NULL;
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) {
        int sh = 0;
        const size_t byte = code_byte(K, n, k, &sh);
        codes[(size_t)n * K + k] = (uint8_t)((h->qw[byte] >> (sh & 7)) & 15);
      }
  }
  if (scales || zeros) {
    if ((scales && !h->scales) || (zeros && !h->zeros)) return SVDQ_ERR_NULL;
    for (int n = 0; n < N; ++n)
      for (int g = 0; g < G; ++g) {
        const size_t i = ((size_t)(n / 16) * G + g) * 16 + n % 16;
        if (scales) scales[(size_t)n * G + g] = h->scales[i];
        if (zeros) zeros[(size_t)n * G + g] = h->zeros[i];
      }
  }
  return SVDQ_OK;
}

}  // extern "C"
