// C-ABI entry points of libsvdq that touch the GPU: argument validation,
// workspace carving and kernel launches on the caller's stream. No
// allocation, no synchronization, nothing printed.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"
#include "svdq_layout.h"

namespace svdq {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950 ready, 2 unsupported
std::atomic<int> g_dev_cus[kMaxDevices];     // compute units of each ready device
std::mutex g_dev_mu;

svdq_status check_device(int* cus = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SVDQ_ERR_DEVICE;
  int s = g_dev_state[dev].load(std::memory_order_acquire);
  if (s == 1) {
    if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    return SVDQ_OK;
  }
  if (s == 2) return SVDQ_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  s = g_dev_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t p;
    bool ok = hipGetDeviceProperties(&p, dev) == hipSuccess &&
              std::strncmp(p.gcnArchName, "gfx950", 6) == 0 && prepare_gemm_mxfp4() == hipSuccess &&
              prepare_gemm_int4() == hipSuccess && prepare_stage1() == hipSuccess;
    s = ok ? 1 : 2;
    if (ok) g_dev_cus[dev].store(p.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(s, std::memory_order_release);
  }
  if (s == 1 && cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return s == 1 ? SVDQ_OK : SVDQ_ERR_DEVICE;
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

svdq_status common_checks(const svdq_layer_desc* d, const svdq_packed* dev, const void* x,
                          int64_t M, const void* ws, size_t ws_bytes) {
  svdq_status st = check_desc(d);
  if (st != SVDQ_OK) return st;
  if (M < 0 || M > (1 << 24)) return SVDQ_ERR_SHAPE;
  // MXFP4 activation scale bytes are addressed with 32-bit stage offsets,
  // the tiled INT4 GEMM's activation codes with 32-bit byte offsets
  if (d->format == SVDQ_FMT_MXFP4_G32 && ((int64_t)d->K + 128) * (round32(M) / 32) >= ((int64_t)1 << 31))
    return SVDQ_ERR_SHAPE;
  if (d->format == SVDQ_FMT_INT4_G64 && round32(M) * d->K > ((int64_t)1 << 33)) return SVDQ_ERR_SHAPE;
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
  a.K = d->K;
  a.r32 = rank32(d->rank);
  a.x = x;
  a.mu = dev->mu;
  a.l1s = dev->l1;
  a.qx = b + L.qx;
  a.sx = b + L.sx;
  a.z = (uint16_t*)(b + L.z);
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  a.flags = int4 ? (uint32_t*)(b + L.flags) : nullptr;
  a.nflags = int4 ? kSplitSlots : 0;
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
  a.N = d->N;
  a.K = d->K;
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
  return a;
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

}  // namespace
}  // namespace svdq

using namespace svdq;

extern "C" {

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
  if (M <= 0 || M > (1 << 24) || round32(M) * d->K > ((int64_t)1 << 33)) return SVDQ_ERR_SHAPE;
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
