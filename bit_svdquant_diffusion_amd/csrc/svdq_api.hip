// C-ABI entry points of libsvdq that touch the GPU: argument validation,
// workspace carving and kernel launches on the caller's stream. No
// allocation, no synchronization, nothing printed.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

namespace svdq {

// Workspace of svdq_linear_forward_noalloc: a library-owned device array, one
// copy per GPU (each device that loads the library holds it until the process
// ends). In host code `scratch` names a host-side stand-in, not device memory:
// the host uses only the per-device address hipGetSymbolAddress returns.
constexpr size_t kNoAllocScratchBytes = (size_t)SVDQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950 ready, 2 unsupported
std::atomic<int> g_dev_cus[kMaxDevices];     // compute units of each ready device
std::atomic<void*> g_dev_scratch[kMaxDevices];   // device address of `scratch` on each ready device
std::mutex g_dev_mu;

// One-time set-up per device, with that device current: the gfx950 check,
// the kernels' LDS attributes and the address of this device's `scratch`.
svdq_status check_device(int* cus = nullptr, void** scratch_ptr = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SVDQ_ERR_DEVICE;
  int s = g_dev_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    std::lock_guard<std::mutex> lock(g_dev_mu);
    s = g_dev_state[dev].load(std::memory_order_acquire);
    if (s == 0) {
      hipDeviceProp_t p;
      void* sp = nullptr;
      bool ok = hipGetDeviceProperties(&p, dev) == hipSuccess &&
                std::strncmp(p.gcnArchName, "gfx950", 6) == 0 && prepare_gemm_mxfp4() == hipSuccess &&
                prepare_gemm_int4() == hipSuccess && prepare_stage1() == hipSuccess && prepare_awq() == hipSuccess &&
                hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) == hipSuccess && sp != nullptr;
      s = ok ? 1 : 2;
      if (ok) {
        g_dev_cus[dev].store(p.multiProcessorCount, std::memory_order_relaxed);
        g_dev_scratch[dev].store(sp, std::memory_order_relaxed);
      }
      g_dev_state[dev].store(s, std::memory_order_release);
    }
  }
  if (s != 1) return SVDQ_ERR_DEVICE;
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (scratch_ptr) *scratch_ptr = g_dev_scratch[dev].load(std::memory_order_relaxed);
  return SVDQ_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

svdq_status check_packed_dev(const svdq_layer_desc* d, const svdq_packed* p) {
  if (!p || !p->mu || !p->qw || !p->sw || !p->bias) return SVDQ_ERR_NULL;
  if (d->rank > 0 && (!p->l1 || !p->l2)) return SVDQ_ERR_NULL;
  if (!aligned16(p->mu) || !aligned16(p->qw) || !aligned16(p->sw) ||
      (d->rank > 0 && (!aligned16(p->l1) || !aligned16(p->l2))))
    return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

// M against the layer: the token limit, and the offsets the kernels address
// with 32 bits (MXFP4 activation scale bytes by stage, the tiled INT4 GEMM's FP6
// activation codes by byte)
svdq_status check_m(const svdq_layer_desc* d, int64_t M) {
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  if (d->format == SVDQ_FMT_MXFP4_G32 && ((int64_t)kpad(d) + 128) * (round32(M) / 32) >= ((int64_t)1 << 31))
    return SVDQ_ERR_SHAPE;
  if (d->format == SVDQ_FMT_INT4_G64 && round32(M) * kpad(d) / 4 * 3 >= ((int64_t)1 << 32)) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

svdq_status common_checks(const svdq_layer_desc* d, const svdq_packed* dev, const void* x,
                          int64_t M, const void* ws, size_t ws_bytes) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  st = check_m(d, M);
  if (st != SVDQ_OK) return st;
  st = check_packed_dev(d, dev);
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  if (!x || !ws) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(ws)) return SVDQ_ERR_SHAPE;
  if (ws_bytes < ws_layout(d, M).total) return SVDQ_ERR_WORKSPACE;
  return SVDQ_OK;
}

Stage1Args stage1_args(const svdq_layer_desc* d, const svdq_packed* dev, const uint16_t* x,
                       int64_t M, void* ws) {
  WsLayout L = ws_layout(d, M);
  uint8_t* b = (uint8_t*)ws;
  Stage1Args a;
  a.fmt = d->format;
  a.M = (int)M;
  a.K = kpad(d);
  a.xk = d->K;
  a.r32 = rank32(d->rank);
  a.x = x;
  a.mu = dev->mu;
  a.l1s = dev->l1;
  a.qx = b + L.qx;
  a.sx = b + L.sx;
  a.z = (uint16_t*)(b + L.z);
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  a.flags = int4 ? (uint32_t*)(b + L.flags) : nullptr;
  a.nflags = int4 ? kSplitCounters : 0;
  a.zp = (float*)(b + L.zp);
  return a;
}

GemmArgs gemm_args(const svdq_layer_desc* d, const svdq_packed* dev, int64_t M, const void* ws,
                   uint16_t* y) {
  WsLayout L = ws_layout(d, M);
  const uint8_t* b = (const uint8_t*)ws;
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.fmt = d->format;
  a.M = (int)M;
  a.N = npad(d);
  a.K = kpad(d);
  a.ldy = d->N;
  a.ldk = d->K;
  a.r32 = rank32(d->rank);
  a.qx = b + L.qx;
  a.sx = b + L.sx;
  a.z = (const uint16_t*)(b + L.z);
  a.qw = dev->qw;
  a.sw = dev->sw;
  a.l2t = dev->l2;
  a.bias = dev->bias;
  a.y = y;
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  a.flags = int4 ? (uint32_t*)(b + L.flags) : nullptr;
  a.part = int4 || M <= kFewTokens ? (float*)(b + L.part) : nullptr;
  a.qx6 = int4_tiled_ws(d, M) ? (uint8_t*)(b + L.x6) : nullptr;
  a.qw6 = int4_tiled_ws(d, M) ? (uint8_t*)(b + L.w6) : nullptr;
  return a;
}

// The MLP pair's workspace: the up layer's, the down layer's, then the
// hidden activation H = GELU(up(x)) as bf16 [M][up N] (composition) or the
// fp32 partial X_hat L1 of the down layer per 256 hidden channels (fused)
struct MlpLayout {
  size_t down, mid, total;
};
MlpLayout mlp_layout(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M) {
  MlpLayout L;
  L.down = align256(ws_layout(up, M).total);
  L.mid = L.down + align256(ws_layout(down, M).total);
  const size_t hid = (size_t)M * up->N * 2;
  const size_t zpart = (size_t)(up->N / 256) * M * rank32(down->rank) * 4;   // at most N / 256 tile columns
  L.total = L.mid + align256(hid > zpart ? hid : zpart);
  return L;
}

svdq_status mlp_shape_checks(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M) {
  if (!up || !down) return SVDQ_ERR_NULL;
  svdq_status st = check_desc(up);
  if (st != SVDQ_OK) return st;
  st = check_desc(down);
  if (st != SVDQ_OK) return st;
  if (down->K != up->N) return SVDQ_ERR_SHAPE;
  st = check_m(up, M);
  if (st != SVDQ_OK) return st;
  return check_m(down, M);
}

// The fused epilogue exists in the tiled GEMMs: both layers in one format,
// the hidden width in whole tile columns (256 channels INT4, 384 MXFP4) and
// whole stage-1 steps (256: the down layer's K needs no padding, which the
// epilogue would not write), more tokens than the weight-streaming kernel
// takes, and partial Z addressed with 32-bit offsets
int mlp_tile_n(const svdq_layer_desc* up) { return up->format == SVDQ_FMT_INT4_G64 ? 256 : 384; }
bool mlp_fusable(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M) {
  return up->format == down->format && up->N % mlp_tile_n(up) == 0 && up->N % 256 == 0 && M > kFewTokens &&
         (uint64_t)(up->N / mlp_tile_n(up)) * M * rank32(down->rank) * 4 < ((uint64_t)1 << 32);
}

bool sync_debug() {
  static const bool v = [] {
    const char* e = std::getenv("SVDQ_SYNC_DEBUG");
    return e && *e == '1';
  }();
  return v;
}

svdq_status after_launch(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return SVDQ_ERR_DEVICE;
  if (sync_debug() && hipStreamSynchronize(s) != hipSuccess) return SVDQ_ERR_DEVICE;
  return SVDQ_OK;
}

// Logical views of a stage-1 workspace, the layouts of svdq_unpack_workspace:
// codes int8 [M][K] (INT4 values, or E2M1 code bits), scales fp32 [M][K/64]
// (INT4) or E8M0 bytes [M][K/32] (MXFP4), Z fp32 [M][rank] (its bf16 values).
// One thread per output element over the three outputs in turn; an absent
// output has no elements. mp = the INT4 scales' row stride, rows32 = the
// MXFP4 scales' row blocks times 32.
__global__ __launch_bounds__(256) void stage1_views_kernel(const uint8_t* __restrict__ qx, const void* __restrict__ sx,
                                                           const uint16_t* __restrict__ zb, int64_t M, int K, int Kp,
                                                           int int4, int r, int r32, int64_t mp, int64_t rows32,
                                                           int8_t* codes, void* scales, float* z, int64_t n_codes,
                                                           int64_t n_scales, int64_t n_z) {
  const int64_t total = n_codes + n_scales + n_z;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n_codes) {
      const int64_t m = i / K;
      const int k = (int)(i - m * K);
      const uint8_t b = qx[f_code_byte(Kp, m, k)];
      const int nib = (k & 1) ? (b >> 4) : (b & 15);
      codes[i] = int4 ? (int8_t)(nib >= 8 ? nib - 16 : nib) : (int8_t)nib;
    } else if (i < n_codes + n_scales) {
      const int64_t j = i - n_codes;
      const int G = int4 ? K / 64 : K / 32;
      const int64_t m = j / G;
      const int g = (int)(j - m * G);
      if (int4)
        static_cast<float*>(scales)[j] = static_cast<const float*>(sx)[(int64_t)g * mp + m];
      else
        static_cast<uint8_t*>(scales)[j] = static_cast<const uint8_t*>(sx)[f_scale_index(rows32, m, g)];
    } else {
      const int64_t j = i - n_codes - n_scales;
      const int64_t m = j / r;
      const int c = (int)(j - m * r);
      z[j] = __uint_as_float((uint32_t)zb[frag16_index(r32, m, c)] << 16);
    }
  }
}

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

svdq_status svdq_stage1_outputs(const svdq_layer_desc* d, const svdq_packed* dev, const uint16_t* x, int64_t M,
                                int8_t* codes, void* scales, float* z, void* ws, size_t ws_bytes, void* stream) {
  // fp32 outputs (Z, INT4 scales) need 4-byte alignment; checked before any work
  if (d && (((uintptr_t)z & 3) || (d->format == SVDQ_FMT_INT4_G64 && ((uintptr_t)scales & 3))))
    return SVDQ_ERR_SHAPE;
  svdq_status st = svdq_stage1(d, dev, x, M, ws, ws_bytes, stream);
  if (st != SVDQ_OK || M == 0 || (!codes && !scales && !z)) return st;
  const WsLayout L = ws_layout(d, M);
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  const int64_t n_codes = codes ? M * d->K : 0;
  const int64_t n_scales = scales ? M * (d->K / (int4 ? 64 : 32)) : 0;
  const int64_t n_z = z ? M * d->rank : 0;
  const int64_t total = n_codes + n_scales + n_z;
  if (total == 0) return SVDQ_OK;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* b = (const uint8_t*)ws;
  hipLaunchKernelGGL(stage1_views_kernel, dim3(grid), dim3(256), 0, s, b + L.qx, (const void*)(b + L.sx),
                     (const uint16_t*)(b + L.z), M, d->K, kpad(d), int4 ? 1 : 0, d->rank, rank32(d->rank),
                     act_rows(M), round32(M), codes, scales, z, n_codes, n_scales, n_z);
  return after_launch(hipGetLastError(), s);
}

svdq_status svdq_stage1(const svdq_layer_desc* d, const svdq_packed* dev, const uint16_t* x,
                        int64_t M, void* ws, size_t ws_bytes, void* stream) {
  svdq_status st = common_checks(d, dev, x, M, ws, ws_bytes);
  if (st != SVDQ_OK || M == 0) return st;
  int cus = 0;
  st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_stage1(stage1_args(d, dev, x, M, ws), cus, s), s);
}

svdq_status svdq_linear_forward(const svdq_layer_desc* d, const svdq_packed* dev,
                                const uint16_t* x, int64_t M, uint16_t* y, void* ws,
                                size_t ws_bytes, void* stream) {
  svdq_status st = common_checks(d, dev, x, M, ws, ws_bytes);
  if (st != SVDQ_OK || M == 0) return st;
  if (!y) return SVDQ_ERR_NULL;
  if (!aligned16(y)) return SVDQ_ERR_SHAPE;
  int cus = 0;
  st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = after_launch(launch_stage1(stage1_args(d, dev, x, M, ws), cus, s), s);
  if (st != SVDQ_OK) return st;
  return after_launch(launch_gemm(gemm_args(d, dev, M, ws, y), cus, s), s);
}

svdq_status svdq_linear_forward_noalloc(const svdq_layer_desc* d, const svdq_packed* dev,
                                        const uint16_t* x, int64_t M, uint16_t* y, void* stream) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  // the workspace this M needs must fit the device array (host arithmetic only)
  if (M > 0 && ws_layout(d, M).total > kNoAllocScratchBytes) return SVDQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (M > 0) {
    st = check_device(nullptr, &ws);
    if (st != SVDQ_OK) return st;
  }
  return svdq_linear_forward(d, dev, x, M, y, ws, kNoAllocScratchBytes, stream);
}

svdq_status svdq_mlp_workspace_bytes(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M,
                                     size_t* out, size_t* down_offset) {
  svdq_status st = mlp_shape_checks(up, down, M);
  if (st != SVDQ_OK) return st;
  if (!out) return SVDQ_ERR_NULL;
  const MlpLayout L = mlp_layout(up, down, M);
  *out = L.total;
  if (down_offset) *down_offset = L.down;
  return SVDQ_OK;
}

svdq_status svdq_mlp_fused(const svdq_layer_desc* up, const svdq_layer_desc* down, int64_t M, int32_t* fused) {
  svdq_status st = mlp_shape_checks(up, down, M);
  if (st != SVDQ_OK) return st;
  if (!fused) return SVDQ_ERR_NULL;
  *fused = mlp_fusable(up, down, M) ? 1 : 0;
  return SVDQ_OK;
}

svdq_status svdq_mlp_forward(const svdq_layer_desc* up, const svdq_packed* dev_up, const svdq_layer_desc* down,
                             const svdq_packed* dev_down, const uint16_t* x, int64_t M, uint16_t* y, void* ws,
                             size_t ws_bytes, int32_t mode, void* stream) {
  svdq_status st = mlp_shape_checks(up, down, M);
  if (st != SVDQ_OK) return st;
  if (mode != SVDQ_MLP_AUTO && mode != SVDQ_MLP_UNFUSED) return SVDQ_ERR_SHAPE;
  st = check_packed_dev(up, dev_up);
  if (st != SVDQ_OK) return st;
  st = check_packed_dev(down, dev_down);
  if (st != SVDQ_OK) return st;
  if (M == 0) return SVDQ_OK;
  if (!x || !y || !ws) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return SVDQ_ERR_SHAPE;
  const MlpLayout L = mlp_layout(up, down, M);
  if (ws_bytes < L.total) return SVDQ_ERR_WORKSPACE;
  int cus = 0;
  st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* b = (uint8_t*)ws;
  uint8_t* wd = b + L.down;
  st = after_launch(launch_stage1(stage1_args(up, dev_up, x, M, b), cus, s), s);
  if (st != SVDQ_OK) return st;
  if (mode == SVDQ_MLP_AUTO && mlp_fusable(up, down, M)) {
    // the up GEMM's epilogue leaves the down layer's stage-1 output in its
    // workspace (codes, scales, per-tile-column partial Z); one small kernel
    // adds the partials into Z
    const WsLayout D = ws_layout(down, M);
    const int r32 = rank32(down->rank);
    GemmArgs a = gemm_args(up, dev_up, M, b, nullptr);
    a.nxt_qx = wd + D.qx;
    a.nxt_sx = wd + D.sx;
    a.nxt_mu = dev_down->mu;
    a.nxt_l1s = dev_down->l1;
    a.nxt_zpart = (float*)(b + L.mid);
    a.nxt_r32 = r32;
    const bool int4 = up->format == SVDQ_FMT_INT4_G64;
    st = after_launch(int4 ? launch_gemm_int4(a, cus, s) : launch_gemm_mxfp4(a, cus, s), s);
    if (st != SVDQ_OK) return st;
    st = after_launch(launch_fused_zsum((const float*)(b + L.mid), up->N / mlp_tile_n(up), (int)M, r32,
                                        (uint16_t*)(wd + D.z), int4 ? (uint32_t*)(wd + D.flags) : nullptr,
                                        int4 ? kSplitCounters : 0, s),
                      s);
  } else {
    uint16_t* hid = (uint16_t*)(b + L.mid);
    st = after_launch(launch_gemm(gemm_args(up, dev_up, M, b, hid), cus, s), s);
    if (st != SVDQ_OK) return st;
    st = after_launch(launch_gelu_bf16(hid, (size_t)M * up->N, s), s);
    if (st != SVDQ_OK) return st;
    st = after_launch(launch_stage1(stage1_args(down, dev_down, hid, M, wd), cus, s), s);
  }
  if (st != SVDQ_OK) return st;
  return after_launch(launch_gemm(gemm_args(down, dev_down, M, wd, y), cus, s), s);
}

svdq_status svdq_awq_forward(const svdq_awq_desc* d, const svdq_awq_packed* dev, const uint16_t* x, int64_t M,
                             uint16_t* y, void* stream) {
  if (!d) return SVDQ_ERR_NULL;
  if (d->K <= 0 || d->N <= 0 || d->K % 128 != 0 || d->K > 4096 || d->N % 16 != 0 || d->N > 65536)
    return SVDQ_ERR_SHAPE;
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  if (!dev || !dev->inv_s || !dev->qw || !dev->scales || !dev->zeros || !dev->bias) return SVDQ_ERR_NULL;
  if (!aligned16(dev->inv_s) || !aligned16(dev->qw) || !aligned16(dev->scales)) return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!x || !y) return SVDQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return SVDQ_ERR_SHAPE;
  int cus = 0;
  svdq_status st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  AwqArgs a;
  a.M = (int)M;
  a.K = d->K;
  a.N = d->N;
  a.x = x;
  a.inv_s = dev->inv_s;
  a.qw = dev->qw;
  a.scales = dev->scales;
  a.zeros = dev->zeros;
  a.bias = dev->bias;
  a.y = y;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_awq(a, cus, s), s);
}

svdq_status svdq_measure_mfma_peak(int32_t kind, int32_t constant_operands, int32_t iters, double* flops,
                                   void* stream) {
  if (!flops) return SVDQ_ERR_NULL;
  if (kind < 0 || kind > 2 || iters < 1 || iters > (1 << 24)) return SVDQ_ERR_SHAPE;
  int cus = 0;
  svdq_status st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_mfma_peak(kind, constant_operands ? 1 : 0, iters, cus, nullptr, s, flops), s);
}

svdq_status svdq_measure_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return SVDQ_OK;
  if (!src || !dst) return SVDQ_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst) || bytes % 16 != 0) return SVDQ_ERR_SHAPE;
  int cus = 0;
  svdq_status st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_copy(src, dst, bytes, cus, s), s);
}

svdq_status svdq_gemm(const svdq_layer_desc* d, const svdq_packed* dev, const void* ws,
                      size_t ws_bytes, int64_t M, uint16_t* y, void* stream) {
  svdq_status st = common_checks(d, dev, ws, M, ws, ws_bytes);
  if (st != SVDQ_OK || M == 0) return st;
  if (!y) return SVDQ_ERR_NULL;
  if (!aligned16(y)) return SVDQ_ERR_SHAPE;
  int cus = 0;
  st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_gemm(gemm_args(d, dev, M, ws, y), cus, s), s);
}

svdq_status svdq_debug_int4_group_sums(const svdq_layer_desc* d, const svdq_packed* dev,
                                       const void* ws, size_t ws_bytes, int64_t M, int64_t m0,
                                       int64_t mc, int64_t n0, int64_t nc, int32_t* p,
                                       void* stream) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (d->format != SVDQ_FMT_INT4_G64) return SVDQ_ERR_FORMAT;
  if (M <= 0 || check_m(d, M) != SVDQ_OK) return SVDQ_ERR_SHAPE;
  st = check_packed_dev(d, dev);
  if (st != SVDQ_OK) return st;
  if (!ws || !p) return SVDQ_ERR_NULL;
  if (!aligned16(ws)) return SVDQ_ERR_SHAPE;
  if (ws_bytes < ws_layout(d, M).total) return SVDQ_ERR_WORKSPACE;
  if (m0 < 0 || mc <= 0 || m0 + mc > M || n0 < 0 || nc <= 0 || n0 + nc > d->N)
    return SVDQ_ERR_SHAPE;
  int cus = 0;
  st = check_device(&cus);
  if (st != SVDQ_OK) return st;
  GemmArgs a = gemm_args(d, dev, M, ws, nullptr);
  a.p = p;
  a.m0 = (int)m0;
  a.mc = (int)mc;
  a.n0 = (int)n0;
  a.nc = (int)nc;
  hipStream_t s = (hipStream_t)stream;
  return after_launch(launch_gemm(a, cus, s), s);
}

}  // extern "C"
