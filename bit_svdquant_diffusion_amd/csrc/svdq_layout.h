// Internal layout helpers shared by the host pack code and the device kernels
// of libsvdq (not part of the public ABI). Everything here is plain integer
// arithmetic on sizes and offsets.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "svdq.h"

// The fragment-order helpers below are also called from device code (the
// GPU-side pack) when this header is compiled by hipcc; g++ sees plain
// inline functions.
#if defined(__HIPCC__)
#define SVDQ_HD __host__ __device__
#else
#define SVDQ_HD
#endif

namespace svdq {

constexpr int kGroupInt4 = 64;    // INT4 scale group along K
constexpr int kBlockMx = 32;      // MXFP4 scale block along K
constexpr int kStepK = 128;       // K per stage-1 step (two INT4 groups)
constexpr int kMaxRank = 128;

inline int rank32(int r) { return (r + 31) / 32 * 32; }
inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// K must hold whole scale groups of the 4-bit GEMM's K step: 64 channels
// (INT4) or 128 (MXFP4); N whole 16-byte runs of bf16 Y (8 channels).
inline svdq_status check_desc(const svdq_layer_desc* d) {
  if (!d) return SVDQ_ERR_NULL;
  if (d->format != SVDQ_FMT_INT4_G64 && d->format != SVDQ_FMT_MXFP4_G32) return SVDQ_ERR_FORMAT;
  const int kq = d->format == SVDQ_FMT_INT4_G64 ? 64 : 128;
  if (d->K <= 0 || d->N <= 0 || d->K % kq != 0 || d->N % 8 != 0) return SVDQ_ERR_SHAPE;
  if (d->K > 65536 || d->N > 65536) return SVDQ_ERR_SHAPE;
  if (d->rank < 0 || d->rank > kMaxRank || d->rank % 16 != 0) return SVDQ_ERR_SHAPE;
  if (d->rank > d->K || d->rank > d->N) return SVDQ_ERR_SHAPE;
  return SVDQ_OK;
}

inline int64_t round32(int64_t v) { return (v + 31) / 32 * 32; }

// Device layouts hold K padded to whole 256-channel stage-1 steps and N
// padded to whole 32-row blocks: the padding's codes, scales, L1 rows, L2
// columns and bias are zero, and stage 1 gives the padded channels of X zero
// codes and scales, so they add nothing. The kernels run on the padded sizes;
// only X's row stride and Y's row stride and width are the layer's own.
inline int kpad(const svdq_layer_desc* d) { return (d->K + 255) / 256 * 256; }
inline int npad(const svdq_layer_desc* d) { return (d->N + 31) / 32 * 32; }

inline size_t scale_bytes(const svdq_layer_desc* d, int64_t rows) {
  return d->format == SVDQ_FMT_INT4_G64 ? (size_t)rows * (kpad(d) / kGroupInt4) * 4
                                        : (size_t)rows * (kpad(d) / kBlockMx);
}
// Row stride of the INT4 activation scales [K/64][act_rows(M)] in the workspace.
inline int64_t act_rows(int64_t M) { return (M + 15) / 16 * 16; }

inline svdq_packed_sizes packed_sizes(const svdq_layer_desc* d) {
  svdq_packed_sizes s;
  s.mu = (size_t)d->K * 4;
  s.l1 = (size_t)kpad(d) * rank32(d->rank) * 2;
  s.l2 = (size_t)npad(d) * rank32(d->rank) * 2;
  s.qw = (size_t)npad(d) * kpad(d) / 2;
  s.sw = scale_bytes(d, npad(d));
  s.bias = (size_t)npad(d) * 2;
  return s;
}

// Stage 1 sums X_hat L1 in K pieces of s1_piece_steps(K) steps of 256
// channels, about twelve pieces whatever K: each wave quarter's partial of a
// piece is complete before it is added, in piece order, and the four quarter
// sums are added last, so a token's Z does not depend on M or on whether a
// workgroup held the whole token group or pieces of it (then a second kernel
// adds the stored partials). The pieces of fewer than 128 token groups are
// dealt over the CUs, so the stored partials cover at most kS1SplitRows rows.
constexpr int kS1Pieces = 12;
inline int s1_piece_steps(int K) { return (K / 256 + kS1Pieces - 1) / kS1Pieces; }
inline int s1_pieces(int K) { return (K / 256 + s1_piece_steps(K) - 1) / s1_piece_steps(K); }
constexpr int64_t kS1SplitRows = 4096;

// INT4 GEMM split of the last tiles over the workgroups (at most
// kSplitSlots of them): two fp32 partial tiles (128 x 256) per workgroup, one
// for the first and one for the last piece of its run, and one ticket counter
// per split tile (fewer than two rounds of tiles, so at most kSplitCounters).
// The few-token GEMM (both formats, M <= kFewTokens) keeps the fp32 partials
// of its K shares in the same area.
constexpr int64_t kFewTokens = 256;
constexpr int kSplitSlots = 256;
constexpr int kSplitPieces = 2;
constexpr int kSplitCounters = 2 * kSplitSlots;
constexpr int kSplitPartBytes = 128 * 256 * 4;
constexpr size_t kPartAreaBytes = (size_t)kSplitPieces * kSplitSlots * kSplitPartBytes;

// Workspace: [qX][sX][Z], each 256-byte aligned, over round32(M) rows. qX and
// Z in fragment order (see below) for both formats; sX fp32 [K/64][act_rows(M)]
// (INT4) or E8M0 bytes in fragment order (MXFP4). INT4 adds the split's flags
// ticket counters (u32 [kSplitCounters], cleared by stage 1) and partial
// tiles (kPartAreaBytes), which MXFP4 with
// M <= kFewTokens has as well (flags unused). Last, with a
// low-rank branch, stage 1's partial Z: fp32, per token group and piece the
// raw MFMA accumulators of its waves, min(round32(M), kS1SplitRows) x
// s1_pieces(K) x 4 x rank32.
//
// INT4 with more than kFewTokens tokens (the tiled GEMM) ends with the codes
// of X and of W once more, as FP6 E2M3 fields (every INT4 code, being in
// [-7, 7], is exact in E2M3), which the GEMM's launch fills from the 4-bit
// codes before every GEMM: per 32-row block and 128-channel stage 3 KiB,
// [group 0 heads][group 1 heads][tails], a lane's head the first 16 of its
// 24 bytes (32 six-bit fields, field i at bit 6 i: channel 32 h + i), its
// tail the last 8 (group 0 at 8 lane, group 1 at 512 + 8 lane).
struct WsLayout {
  size_t qx, sx, z, flags, part, zp, x6, w6, total;
};
inline bool int4_tiled_ws(const svdq_layer_desc* d, int64_t M) {
  return d->format == SVDQ_FMT_INT4_G64 && M > kFewTokens;
}
inline WsLayout ws_layout(const svdq_layer_desc* d, int64_t M) {
  WsLayout w;
  const bool int4 = d->format == SVDQ_FMT_INT4_G64;
  const int64_t rows = round32(M);
  w.qx = 0;
  w.sx = align256((size_t)rows * kpad(d) / 2);
  w.z = w.sx + align256(scale_bytes(d, int4 ? act_rows(M) : rows));
  w.flags = w.z + align256((size_t)rows * rank32(d->rank) * 2);
  w.part = w.flags + (int4 ? align256((size_t)kSplitCounters * 4) : 0);
  w.zp = w.part + (int4 || M <= kFewTokens ? kPartAreaBytes : 0);
  w.x6 = align256(w.zp + (size_t)s1_pieces(kpad(d)) * (rows < kS1SplitRows ? rows : kS1SplitRows) * 4 * rank32(d->rank) * 4);
  const bool fp6 = int4_tiled_ws(d, M);
  w.w6 = w.x6 + (fp6 ? align256((size_t)rows * kpad(d) / 4 * 3) : 0);
  w.total = w.w6 + (fp6 ? align256((size_t)npad(d) * kpad(d) / 4 * 3) : 0);
  return w;
}

// Fragment order of 4-bit codes (both formats): rows in blocks of 32, K in
// steps of 64; each (block, step) is 1 KiB = 64 lanes x 16 bytes, lane
// l = 32h + r holding row 32*block + r, channels 64*step + 32h + [0, 32) (even
// channel in the low nibble). One (block, step) is one MXFP4 MFMA operand of
// one wave, or one INT4 group of 32 rows (two i8 MFMA operands once widened).
SVDQ_HD inline size_t f_code_byte(int K, int64_t row, int k) {
  const int64_t b = row / 32;
  const int r = (int)(row % 32), S = k / 64, h = (k % 64) / 32, j = k % 32;
  return (((size_t)b * (K / 64) + S) * 64 + (32 * h + r)) * 16 + j / 2;
}
// Fragment order of a bf16 operand with rank32 columns (Z = X_hat L1 and
// L2^T): rows in blocks of 32, columns in steps of 16; each
// (block, step) is 1 KiB = 64 lanes x 8 bf16, lane l = 32h + r holding row
// 32*block + r, columns 16*step + 8h + [0, 8). Returns an element index.
SVDQ_HD inline size_t frag16_index(int r32, int64_t row, int col) {
  const int64_t b = row / 32;
  const int r = (int)(row % 32), c = col / 16, h = (col % 16) / 8, j = col % 8;
  return (((size_t)b * (r32 / 16) + c) * 64 + (32 * h + r)) * 8 + j;
}

// Fragment order of MXFP4 scale bytes: [K/128 stage][rows32/32 block][64 lanes][2];
// lane l = 32h + r of block b at stage st holds the bytes of the 32-channel
// blocks kb = 4 st + 2 step + h (step = 0, 1) of row 32 b + r.
SVDQ_HD inline size_t f_scale_index(int64_t rows32, int64_t row, int kb) {
  const int st = kb / 4, step = (kb % 4) / 2, h = kb % 2;
  return (((size_t)st * (rows32 / 32) + row / 32) * 64 + (32 * h + row % 32)) * 2 + step;
}

// L1 device layout: [K/256][4 quarters][rank32/16][t=2][lane=64][8] bf16 where
// lane = 16j + c holds L1[256 s + 64 w + 16 j + 8 t + e][16 cb + c], e = 0..7:
// the B operand of stage-1 MFMA t of wave w in step s for the 16 columns cb.
inline size_t l1_index(int K, int r32, int k, int col) {
  (void)K;
  const int s = k / 256, w = (k % 256) / 64, j = (k % 64) / 16, t = (k % 16) / 8, e = k % 8;
  const int cb = col / 16, c = col % 16;
  return (((((size_t)s * 4 + w) * (r32 / 16) + cb) * 2 + t) * 64 + (16 * j + c)) * 8 + e;
}


}  // namespace svdq
