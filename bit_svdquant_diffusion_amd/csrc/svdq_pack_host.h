// Host-side pieces of the pack shared by the host pack (svdq_pack.cpp) and
// the GPU-side pack (svdq_pack_gpu.hip): the randomized truncated SVD over
// two panel products, the smoothing multipliers, bf16 rounding and the
// device layout of the low-rank factors. Internal, not part of the ABI.
#pragma once
#include <stdint.h>

#include <functional>
#include <vector>

#include "svdq.h"

namespace svdq {

// out = W_hat in (in [N][L] -> out [K][L]) or W_hat^T in (in [K][L] -> out [N][L])
using PanelOp = std::function<svdq_status(const double* in, double* out)>;

// Top-r factors L1 [K][r] = U_r Sigma_r, L2 [r][N] = V_r^T (fp64) of the K x N
// matrix that the two products apply; the panel width is r + max(16, r / 2)
// (at most min(K, N)).
svdq_status truncated_svd_ops(int64_t K, int64_t N, int r, uint64_t seed, const PanelOp& AX, const PanelOp& AtX,
                              std::vector<double>& L1, std::vector<double>& L2);

// mu_k = fl32(1 / lambda_k), lambda_k = ax_k^alpha / aw_k^(1 - alpha) in fp64
// (sqrt(ax / aw) at alpha = 1/2), 1 where either is 0.
svdq_status smoothing_mu(int K, const float* ax, const float* aw, double alpha, float* mu);

uint16_t bf16_from_double(double v);
double bf16_to_double(uint16_t b);

// L1 [K][rank] and L2 [rank][N] (bf16 bits, logical) in the packed layer's
// device layout, padding zero.
void factor_layout(const svdq_layer_desc* d, const uint16_t* l1b, const uint16_t* l2b, uint16_t* l1_out,
                   uint16_t* l2_out);

}  // namespace svdq
