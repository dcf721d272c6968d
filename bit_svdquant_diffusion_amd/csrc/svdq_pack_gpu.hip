// GPU-side pack of an SVDQuant layer and the calibrated smoothing strength
// (aiflownews.com, "What SVDQuant actually does": the method needs a
// calibration pass on representative data and then the quantization; "Native
// Diffusers integration and the new workflow": calibrate, quantize, package).
//
// The pack's steps are those of svdq_pack_weights; what is O(K N) or
// O(K N r) runs on the GPU:
//   - the column maxima of W;
//   - the randomized SVD's products with W_hat = diag(1/mu) W (fp64, split
//     over the reduction dimension, the splits added in order);
//   - the residual R = fl32(W_hat - L1 L2) against the bf16 factors (fp64,
//     terms added in increasing rank index, no fused multiply-add: the host
//     pack's arithmetic, so the codes are the same bits) and its 4-bit
//     quantization straight into the device layout.
// The panel orthonormalizations, the small Jacobi SVD and the device layout
// of the factors run on the host, as in the host pack.
//
// The calibration packs the layer for each strength alpha of a grid
// (lambda_k = max|X_k|^alpha / max|W_k|^(1 - alpha)), runs the forward on the
// calibration rows and keeps the alpha whose output is closest to X W^T + b
// (squared error, fp64).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "svdq_device.h"
#include "svdq_internal.h"
#include "svdq_layout.h"
#include "svdq_pack_host.h"

namespace svdq {

namespace {

constexpr int kPT = 64;   // panel tile: rows, columns and reduction step

// part[c][i][j] = sum over p of chunk c of A(i, p) B(p, j) with, for the
// product with W_hat (TRANS false, i over K, p over N): A(i, p) = w[p][i],
// B = X; for the product with W_hat^T (TRANS true, i over N, p over K):
// A(i, p) = w[i][p], B(p, j) = X[p][j] / mu_p. w is fp32 [N][K].
template <bool TRANS>
__global__ __launch_bounds__(256) void panel_kernel(const float* __restrict__ w, int K, int N,
                                                    const double* __restrict__ X, int L,
                                                    const float* __restrict__ mu, int chunk, double* __restrict__ part) {
  __shared__ double As[kPT][kPT + 1];
  __shared__ double Bs[kPT][kPT + 1];
  const int rows = TRANS ? N : K, P = TRANS ? K : N;
  const int i0 = blockIdx.x * kPT, j0 = blockIdx.y * kPT, c = blockIdx.z;
  const int pb = c * chunk, pe = min(P, pb + chunk);
  const int t = threadIdx.x, ti = t >> 2, tj = t & 3;
  double acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.0;
  for (int p0 = pb; p0 < pe; p0 += kPT) {
#pragma unroll 4
    for (int e = 0; e < 16; ++e) {
      const int idx = t + 256 * e;
      if (TRANS) {
        const int ii = idx / kPT, pp = idx % kPT;
        const int i = i0 + ii, p = p0 + pp;
        As[ii][pp] = (i < rows && p < pe) ? (double)w[(size_t)i * K + p] : 0.0;
      } else {
        const int pp = idx / kPT, ii = idx % kPT;
        const int i = i0 + ii, p = p0 + pp;
        As[ii][pp] = (i < rows && p < pe) ? (double)w[(size_t)p * K + i] : 0.0;
      }
      const int pp = idx / kPT, jj = idx % kPT;
      const int p = p0 + pp, j = j0 + jj;
      double b = (p < pe && j < L) ? X[(size_t)p * L + j] : 0.0;
      if (TRANS && p < pe && j < L) b = b / (double)mu[p];
      Bs[pp][jj] = b;
    }
    __syncthreads();
#pragma unroll 8
    for (int pp = 0; pp < kPT; ++pp) {
      const double a = As[ti][pp];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc[u] += a * Bs[pp][tj + 4 * u];
    }
    __syncthreads();
  }
  const int i = i0 + ti;
  if (i < rows) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + tj + 4 * u;
      if (j < L) part[((size_t)c * rows + i) * L + j] = acc[u];
    }
  }
}

// out[i][j] = sum over chunks in order of part[c][i][j], divided by mu_i for
// the product with W_hat (its rows are the smoothed channels)
__global__ void panel_reduce(const double* __restrict__ part, int chunks, int rows, int L,
                             const float* __restrict__ mu, double* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * L) return;
  double s = part[idx];
  for (int c = 1; c < chunks; ++c) s += part[(size_t)c * rows * L + idx];
  if (mu) s = s / (double)mu[idx / L];
  out[idx] = s;
}

// aw[k] = max_n |w[n][k]|
__global__ void colmax_f32(const float* __restrict__ w, int N, int K, float* __restrict__ aw) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  float m = 0.f;
  for (int n = 0; n < N; ++n) m = fmaxf(m, fabsf(w[(size_t)n * K + k]));
  aw[k] = m;
}

// ax[k] = max_m |x[m][k]| over bf16 rows
__global__ void colmax_bf16(const uint16_t* __restrict__ x, int M, int K, float* __restrict__ ax) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  float m = 0.f;
  for (int r = 0; r < M; ++r) m = fmaxf(m, fabsf(__uint_as_float((uint32_t)x[(size_t)r * K + k] << 16)));
  ax[k] = m;
}

__global__ void fill_u32(uint32_t* __restrict__ p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// E2M1 code of an exact real, nearest with ties to the even mantissa bit,
// saturating at 6 (the midpoints of the E2M1 grid decide)
__device__ __forceinline__ uint32_t e2m1_exact(double v) {
  const double a = fabs(v);
  uint32_t c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return signbit(v) ? (c | 8u) : c;
}

// One thread per output row n and scale group g of the layer (64 channels
// INT4, 32 MXFP4): the residual against the bf16 factors (L1d [K][r], L2d
// [r][N] hold their values in fp64), then its codes and scale written in the
// device layout. Workgroups cover 64 consecutive rows of one group, so the
// L1 row reads are shared and the L2 reads coalesce.
template <int FMT>
__global__ __launch_bounds__(64) void residual_quant(const float* __restrict__ w, const float* __restrict__ mu,
                                                     const double* __restrict__ L1d, const double* __restrict__ L2d,
                                                     int K, int N, int r, int Kp, int Np, uint8_t* __restrict__ qw,
                                                     void* __restrict__ sw) {
  constexpr bool INT4 = FMT == SVDQ_FMT_INT4_G64;
  constexpr int GS = INT4 ? 64 : 32;
  const int n = blockIdx.x * 64 + threadIdx.x, g = blockIdx.y;
  if (n >= N) return;
  float rv[GS];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < GS; ++j) {
    const int k = g * GS + j;
    const double what = (double)w[(size_t)n * K + k] / (double)mu[k];
    double acc = 0.0;
    for (int i = 0; i < r; ++i) acc = __dadd_rn(acc, __dmul_rn(L1d[(size_t)k * r + i], L2d[(size_t)i * N + n]));
    rv[j] = (float)__dsub_rn(what, acc);
    amax = fmaxf(amax, fabsf(rv[j]));
  }
  uint32_t words[GS / 8];
#pragma unroll
  for (int q = 0; q < GS / 8; ++q) words[q] = 0u;
  if constexpr (INT4) {
    const float s = amax / 7.0f;   // IEEE-rounded division
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      int q = 0;
      if (s != 0.f) q = (int)fmin(7.0, fmax(-7.0, rint((double)rv[j] / (double)s)));
      words[j / 8] |= ((uint32_t)q & 15u) << (4 * (j % 8));
    }
    reinterpret_cast<float*>(sw)[(size_t)g * Np + n] = s;
  } else {
    int e = -127;
    if (amax > 0.f) {
      int E;
      frexp((double)amax, &E);   // amax = f 2^E, f in [0.5, 1)
      e = max(-127, min(127, (E - 1) - 2));
    }
#pragma unroll
    for (int j = 0; j < GS; ++j) words[j / 8] |= e2m1_exact(ldexp((double)rv[j], -e)) << (4 * (j % 8));
    reinterpret_cast<uint8_t*>(sw)[f_scale_index(Np, n, g)] = (uint8_t)(e + 127);
  }
  // 32 channels a lane in fragment order: 16 contiguous bytes
#pragma unroll
  for (int h = 0; h < GS / 32; ++h)
    *reinterpret_cast<u32x4*>(qw + f_code_byte(Kp, n, g * GS + 32 * h)) =
        u32x4{words[4 * h], words[4 * h + 1], words[4 * h + 2], words[4 * h + 3]};
}

// yref[m][n] = sum_k x[m][k] w[n][k] + b[n] (fp64); one workgroup per row m
// and 256 outputs (the row of x is read by all of them, from cache)
__global__ __launch_bounds__(256) void ref_kernel(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ bias, int K, int N,
                                                  double* __restrict__ yref) {
  const int m = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  double acc = 0.0;
  const float* wr = w + (size_t)n * K;
  const uint16_t* xr = x + (size_t)m * K;
  for (int k = 0; k < K; ++k) acc += (double)__uint_as_float((uint32_t)xr[k] << 16) * (double)wr[k];
  yref[(size_t)m * N + n] = acc + (bias ? (double)bias[n] : 0.0);
}

// loss[m] = sum_n (y[m][n] - yref[m][n])^2, a fixed reduction order
__global__ __launch_bounds__(256) void row_loss(const uint16_t* __restrict__ y, const double* __restrict__ yref,
                                                int N, double* __restrict__ loss) {
  __shared__ double red[256];
  const int m = blockIdx.x;
  double s = 0.0;
  for (int n = threadIdx.x; n < N; n += 256) {
    const double d = (double)__uint_as_float((uint32_t)y[(size_t)m * N + n] << 16) - yref[(size_t)m * N + n];
    s += d * d;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[m] = red[0];
}

int panel_width(const svdq_layer_desc* d) {
  const int r = d->rank;
  return (int)std::min<int64_t>(r + std::max(16, r / 2), std::min(d->K, d->N));
}
// split of the reduction dimension P for `rows` output rows: about 512 workgroups
int panel_chunks(int rows, int P, int L) {
  const int tiles = ((rows + kPT - 1) / kPT) * ((L + kPT - 1) / kPT);
  int c = std::max(1, std::min(16, 512 / std::max(1, tiles)));
  return std::min(c, std::max(1, (P + kPT - 1) / kPT));
}

struct PackWs {
  size_t aw, xin, xout, part, l1d, l2d, total;
};
PackWs pack_ws(const svdq_layer_desc* d) {
  const int K = d->K, N = d->N, L = d->rank > 0 ? panel_width(d) : 1, r = std::max(d->rank, 1);
  const size_t rowsmax = (size_t)std::max(K, N);
  const size_t part = std::max((size_t)panel_chunks(K, N, L) * K, (size_t)panel_chunks(N, K, L) * N) * L * 8;
  PackWs p;
  p.aw = 0;
  p.xin = align256((size_t)K * 4);
  p.xout = p.xin + align256(rowsmax * L * 8);
  p.part = p.xout + align256(rowsmax * L * 8);
  p.l1d = p.part + align256(part);
  p.l2d = p.l1d + align256((size_t)K * r * 8);
  p.total = p.l2d + align256((size_t)r * N * 8);
  return p;
}

struct CalWs {
  size_t pack, fwd, y, yref, loss, ax, total;
};
CalWs cal_ws(const svdq_layer_desc* d, int64_t m) {
  CalWs c;
  c.pack = 0;
  c.fwd = align256(pack_ws(d).total);
  c.y = c.fwd + align256(ws_layout(d, m).total);
  c.yref = c.y + align256((size_t)m * d->N * 2);
  c.loss = c.yref + align256((size_t)m * d->N * 8);
  c.ax = c.loss + align256((size_t)m * 8);
  c.total = c.ax + align256((size_t)d->K * 4);
  return c;
}

svdq_status hip_ok(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_DEVICE; }

// The whole pack into dev_out; synchronizes the stream.
svdq_status pack_gpu(const svdq_layer_desc* d, const float* w, const float* bias, const float* ax_dev, double alpha,
                     uint64_t seed, svdq_packed* out, uint8_t* ws, hipStream_t st) {
  const int K = d->K, N = d->N, r = d->rank, Kp = kpad(d), Np = npad(d);
  const PackWs P = pack_ws(d);
  float* aw = (float*)(ws + P.aw);
  // 1. smoothing multipliers (the column maxima on the GPU, the rule on the host)
  hipLaunchKernelGGL(colmax_f32, dim3((K + 255) / 256), dim3(256), 0, st, w, N, K, aw);
  std::vector<float> h_aw(K), h_ax(K), h_mu(K);
  if (hipMemcpyAsync(h_aw.data(), aw, (size_t)K * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(h_ax.data(), ax_dev, (size_t)K * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return SVDQ_ERR_DEVICE;
  for (int k = 0; k < K; ++k)
    if (!std::isfinite(h_aw[k]) || !std::isfinite(h_ax[k])) return SVDQ_ERR_NUMERIC;
  svdq_status s = smoothing_mu(K, h_ax.data(), h_aw.data(), alpha, h_mu.data());
  if (s != SVDQ_OK) return s;
  if (hipMemcpyAsync(out->mu, h_mu.data(), (size_t)K * 4, hipMemcpyHostToDevice, st) != hipSuccess)
    return SVDQ_ERR_DEVICE;
  // 2. low-rank factors: randomized SVD with the products on the GPU
  std::vector<uint16_t> l1b((size_t)K * r), l2b((size_t)r * N);
  if (r > 0) {
    const int L = panel_width(d);
    double* xin = (double*)(ws + P.xin);
    double* xout = (double*)(ws + P.xout);
    double* part = (double*)(ws + P.part);
    auto product = [&](bool trans, const double* in, double* outp) -> svdq_status {
      const int rows = trans ? N : K, Pd = trans ? K : N;
      const int chunks = panel_chunks(rows, Pd, L);
      const int chunk = ((Pd + chunks - 1) / chunks + kPT - 1) / kPT * kPT;
      const int used = (Pd + chunk - 1) / chunk;
      if (hipMemcpyAsync(xin, in, (size_t)Pd * L * 8, hipMemcpyHostToDevice, st) != hipSuccess) return SVDQ_ERR_DEVICE;
      const dim3 grid((rows + kPT - 1) / kPT, (L + kPT - 1) / kPT, used);
      if (trans)
        hipLaunchKernelGGL(panel_kernel<true>, grid, dim3(256), 0, st, w, K, N, xin, L, out->mu, chunk, part);
      else
        hipLaunchKernelGGL(panel_kernel<false>, grid, dim3(256), 0, st, w, K, N, xin, L, out->mu, chunk, part);
      const size_t n = (size_t)rows * L;
      hipLaunchKernelGGL(panel_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, used, rows, L,
                         trans ? nullptr : out->mu, xout);
      if (hipGetLastError() != hipSuccess ||
          hipMemcpyAsync(outp, xout, n * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
          hipStreamSynchronize(st) != hipSuccess)
        return SVDQ_ERR_DEVICE;
      return SVDQ_OK;
    };
    std::vector<double> L1, L2;
    s = truncated_svd_ops(
        K, N, r, seed, [&](const double* in, double* o) { return product(false, in, o); },
        [&](const double* in, double* o) { return product(true, in, o); }, L1, L2);
    if (s != SVDQ_OK) return s;
    for (size_t i = 0; i < L1.size(); ++i) l1b[i] = bf16_from_double(L1[i]);
    for (size_t i = 0; i < L2.size(); ++i) l2b[i] = bf16_from_double(L2[i]);
  }
  // 3. factors and bias in device layout (host), the residual's codes (GPU)
  const svdq_packed_sizes sz = packed_sizes(d);
  std::vector<uint16_t> hl1(sz.l1 / 2), hl2(sz.l2 / 2), hb(sz.bias / 2, 0);
  if (r > 0) factor_layout(d, l1b.data(), l2b.data(), hl1.data(), hl2.data());
  std::vector<float> hbias(N, 0.f);
  if (bias && hipMemcpyAsync(hbias.data(), bias, (size_t)N * 4, hipMemcpyDeviceToHost, st) != hipSuccess)
    return SVDQ_ERR_DEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return SVDQ_ERR_DEVICE;
  for (int n = 0; n < N; ++n) {
    if (!std::isfinite(hbias[n])) return SVDQ_ERR_NUMERIC;
    hb[n] = bf16_from_double((double)hbias[n]);
  }
  const int rr = std::max(r, 1);
  std::vector<double> d1((size_t)K * rr, 0.0), d2((size_t)rr * N, 0.0);
  for (size_t i = 0; i < l1b.size(); ++i) d1[i] = bf16_to_double(l1b[i]);
  for (size_t i = 0; i < l2b.size(); ++i) d2[i] = bf16_to_double(l2b[i]);
  double* l1d = (double*)(ws + P.l1d);
  double* l2d = (double*)(ws + P.l2d);
  if ((r > 0 && (hipMemcpyAsync(out->l1, hl1.data(), sz.l1, hipMemcpyHostToDevice, st) != hipSuccess ||
                 hipMemcpyAsync(out->l2, hl2.data(), sz.l2, hipMemcpyHostToDevice, st) != hipSuccess)) ||
      hipMemcpyAsync(out->bias, hb.data(), sz.bias, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(l1d, d1.data(), d1.size() * 8, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(l2d, d2.data(), d2.size() * 8, hipMemcpyHostToDevice, st) != hipSuccess)
    return SVDQ_ERR_DEVICE;
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)((sz.qw / 4 + 255) / 256)), dim3(256), 0, st, (uint32_t*)out->qw, sz.qw / 4);
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)((sz.sw / 4 + 255) / 256)), dim3(256), 0, st, (uint32_t*)out->sw, sz.sw / 4);
  if (d->format == SVDQ_FMT_INT4_G64)
    hipLaunchKernelGGL(residual_quant<SVDQ_FMT_INT4_G64>, dim3((N + 63) / 64, K / 64), dim3(64), 0, st, w, out->mu,
                       l1d, l2d, K, N, r, Kp, Np, out->qw, out->sw);
  else
    hipLaunchKernelGGL(residual_quant<SVDQ_FMT_MXFP4_G32>, dim3((N + 63) / 64, K / 32), dim3(64), 0, st, w, out->mu,
                       l1d, l2d, K, N, r, Kp, Np, out->qw, out->sw);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return SVDQ_ERR_DEVICE;
  return SVDQ_OK;
}

bool packed_dev_ok(const svdq_layer_desc* d, const svdq_packed* p) {
  return p && p->mu && p->qw && p->sw && p->bias && (d->rank == 0 || (p->l1 && p->l2));
}

}  // namespace

}  // namespace svdq

using namespace svdq;

extern "C" {

svdq_status svdq_pack_gpu_workspace_bytes(const svdq_layer_desc* d, size_t* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  *out = pack_ws(d).total;
  return SVDQ_OK;
}

svdq_status svdq_pack_weights_gpu(const svdq_layer_desc* d, const float* w_lin, const float* bias,
                                  const float* act_absmax, float alpha, uint64_t seed, svdq_packed* dev_out,
                                  void* workspace, size_t ws_bytes, void* stream) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!w_lin || !act_absmax || !workspace || !packed_dev_ok(d, dev_out)) return SVDQ_ERR_NULL;
  if (!(alpha >= 0.f && alpha <= 1.f)) return SVDQ_ERR_SHAPE;
  if (ws_bytes < pack_ws(d).total) return SVDQ_ERR_WORKSPACE;
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess ||
      std::strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return SVDQ_ERR_DEVICE;
  return pack_gpu(d, w_lin, bias, act_absmax, (double)alpha, seed, dev_out, (uint8_t*)workspace,
                  (hipStream_t)stream);
}

svdq_status svdq_calibrate_workspace_bytes(const svdq_layer_desc* d, int64_t m_cal, size_t* out) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  if (m_cal <= 0 || m_cal > 65536) return SVDQ_ERR_SHAPE;
  *out = cal_ws(d, m_cal).total;
  return SVDQ_OK;
}

svdq_status svdq_calibrate_alpha(const svdq_layer_desc* d, const float* w_lin, const float* bias,
                                 const uint16_t* x_cal, int64_t m_cal, const float* alphas, int32_t n_alpha,
                                 uint64_t seed, float* alpha_out, double* losses_out, svdq_packed* dev_out,
                                 void* workspace, size_t ws_bytes, void* stream) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (!w_lin || !x_cal || !alphas || !workspace || !packed_dev_ok(d, dev_out)) return SVDQ_ERR_NULL;
  if (m_cal <= 0 || m_cal > 65536 || n_alpha <= 0 || n_alpha > 64) return SVDQ_ERR_SHAPE;
  for (int i = 0; i < n_alpha; ++i)
    if (!(alphas[i] >= 0.f && alphas[i] <= 1.f)) return SVDQ_ERR_SHAPE;
  const CalWs C = cal_ws(d, m_cal);
  if (ws_bytes < C.total) return SVDQ_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  float* ax = (float*)(ws + C.ax);
  uint16_t* y = (uint16_t*)(ws + C.y);
  double* yref = (double*)(ws + C.yref);
  double* loss = (double*)(ws + C.loss);
  const int K = d->K, N = d->N;
  hipLaunchKernelGGL(colmax_bf16, dim3((K + 255) / 256), dim3(256), 0, s, x_cal, (int)m_cal, K, ax);
  hipLaunchKernelGGL(ref_kernel, dim3((N + 255) / 256, (unsigned)m_cal), dim3(256), 0, s, x_cal, w_lin, bias, K, N,
                     yref);
  if (hipGetLastError() != hipSuccess) return SVDQ_ERR_DEVICE;
  std::vector<double> rows(m_cal);
  int best = -1;
  double best_loss = 0.0;
  for (int i = 0; i < n_alpha; ++i) {
    st = pack_gpu(d, w_lin, bias, ax, (double)alphas[i], seed, dev_out, ws + C.pack, s);
    if (st != SVDQ_OK) return st;
    st = svdq_linear_forward(d, dev_out, x_cal, m_cal, y, ws + C.fwd, C.y - C.fwd, stream);
    if (st != SVDQ_OK) return st;
    hipLaunchKernelGGL(row_loss, dim3((unsigned)m_cal), dim3(256), 0, s, y, yref, N, loss);
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(rows.data(), loss, (size_t)m_cal * 8, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return SVDQ_ERR_DEVICE;
    double l = 0.0;
    for (int64_t m = 0; m < m_cal; ++m) l += rows[m];
    if (losses_out) losses_out[i] = l;
    if (best < 0 || l < best_loss) {
      best = i;
      best_loss = l;
    }
  }
  if (alpha_out) *alpha_out = alphas[best];
  // the kept layer: packed again with the best alpha unless it was the last
  if (best != n_alpha - 1) return pack_gpu(d, w_lin, bias, ax, (double)alphas[best], seed, dev_out, ws + C.pack, s);
  return SVDQ_OK;
}

}  // extern "C"
