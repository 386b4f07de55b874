// kq_internal.h -- layout constants and launch entry points shared by the
// C-ABI wrapper (kq_api.cpp) and the HIP kernels (kq_kernels.hip).
#pragma once
#include <stdint.h>
#include <stddef.h>

#include "kq.h"

namespace kq {

constexpr int64_t kQK = 256;          // weights per Q4_K super-block
constexpr int64_t kBlockBytes = 144;  // bytes per super-block
constexpr int kMaxRows = 16;          // activation rows per MFMA slice (block size of the draft)
constexpr int kMaxTreeRows = 64;      // activation rows per call: up to 4 slices (token-tree verify)
// 16-row slices staged for m activation rows: one per 16 rows or part of
// them (1 to 4); a launch runs all of them in one pass over the weights
constexpr int row_slices(int m) { return (m + 15) / 16; }
constexpr int kMaxGroup = 8;          // matrices per grouped launch
// Rows per row group of a chain launch (kq_chain_kernel's compute waves times
// 16-row tiles)
constexpr int kChainRows = 128;

// Tiled weight layout (see kq_tile_weights in kq.h): 2,304-byte records of
// one block of one 16-row tile: headers, then the two quant halves in lane
// order.
constexpr int64_t kTileBlockBytes = 16 * kBlockBytes;  // 2,304
constexpr int64_t kTileQ0 = 256;
constexpr int64_t kTileQ1 = 1280;

// Weight formats of the main kernel: Q4_K (row-major or tiled), Q5_K and
// Q6_K (tiled only; kq_tile_weights_fmt). Their tiled records keep the Q4_K
// lane order for the low four bits of every weight (the same staged
// activations serve every format):
//   Q5_K (2,816 B): headers as Q4_K | quant halves as Q4_K | 64 lanes x 8 B
//                   of fifth bits (kTileQH)
//   Q6_K (3,360 B): 64 lanes x 4 scale bytes | low-nibble halves as Q4_K |
//                   64 lanes x 16 B of 2-bit high parts (kTileQH) | 16 fp16 d
//                   (kTileQ6D)
constexpr int kFmtQ4 = 0, kFmtQ5 = 1, kFmtQ6 = 2;
constexpr int64_t kBlockBytesQ5 = 176;
constexpr int64_t kBlockBytesQ6 = 210;
constexpr int64_t kTileQH = 2304;
constexpr int64_t kTileQ6D = 3328;
constexpr int64_t fmt_block_bytes(int fmt) {
  return fmt == kFmtQ6 ? kBlockBytesQ6 : fmt == kFmtQ5 ? kBlockBytesQ5 : kBlockBytes;
}
// format of a layout code (-1 for an unknown code)
constexpr int layout_fmt(int layout) {
  return layout == KQ_LAYOUT_ROWS || layout == KQ_LAYOUT_TILED16 ? kFmtQ4
         : layout == KQ_LAYOUT_Q5K_TILED16                       ? kFmtQ5
         : layout == KQ_LAYOUT_Q6K_TILED16                       ? kFmtQ6
                                                                 : -1;
}

// Staged activations, one record per 256-column block and 16-row slice
// (records [block][slice]; a call of m rows has row_slices(m) slices; each
// row scaled by a power of two 2^e chosen from that row's largest magnitude
// in the block):
//   XA  [8 k-steps][hi,lo][64 lanes][8 x fp16]  16,384 B  MFMA A operand
//   XSB [64 lanes][4 x fp16]                       512 B  sub-block sums (min-term A operand)
//   XI  [16] fp32                                    64 B  per-row 2^-e
constexpr int64_t kXaBytes = 16384;
constexpr int64_t kXsbOffset = 16384;
constexpr int64_t kXiOffset = 16384 + 512;
constexpr int64_t kStageBytes = 16384 + 512 + 64;  // 16,960 B per block (16-B aligned)

// Scratch area of the main kernel (control words zero between calls; every
// launch leaves them zero again):
//   0          done counter (u32, verify)
//   128        grid-barrier arrival count (u32, chain launches)
//   256        barrier time-out flag (u32, chain launches; sticky: set only
//              when a barrier wait gave up, cleared by kq_workspace_init)
//   384        launch epoch (u32, chain launches; +1 per completed launch)
//   cnt_off    per-row-group arrival counters [n_groups], one u32 per
//              128-byte line (kCntStride words apart) so that the atomics of
//              different groups do not queue on one line
//   keys_off   per-workgroup argmax keys [n_wg][kMaxTreeRows] (u64)
//   part_off   partial sums [n_wg][2][rows per group][16 * slices] fp32
constexpr int64_t kBarOff = KQ_CHAIN_BARRIER_OFFSET;
constexpr int64_t kErrOff = KQ_CHAIN_ERROR_OFFSET;
constexpr int64_t kEpochOff = 384;
constexpr int64_t kCntOff = 512;
constexpr int kCntStride = 32;

// Work decomposition. A row group is 16 * waves * tpw consecutive output rows
// of one matrix; a unit is one row group times one 256-column block. The
// launch has n_wg persistent workgroups; workgroup p processes the units
// [p * base + min(p, rem), +base + (p < rem)) of the row-group-major unit
// order, base = units / n_wg, rem = units % n_wg.
struct Geometry {
  int count;      // matrices in the launch (same n, k, activations)
  int waves;      // waves per workgroup (4 or 8)
  int tpw;        // 16-row tiles per wave (1 or 2)
  int bi;         // units between workgroup barriers (1, 2 or 4; LDS ring of 2 bi blocks)
  int depth;      // weight register sets (prefetch depth + 1: 4 or 8)
  int ms;         // 16-row activation slices of the launch (1 to 4)
  int rows;       // rows per row group = 16 * waves * tpw
  int n_wg_per;   // row groups per matrix
  int n_groups;   // row groups in total = count * n_wg_per
  int kb;         // 256-column blocks per row
  int64_t units;  // n_groups * kb
  int n_wg;       // persistent workgroups (<= units)
};

struct ScratchLayout {
  size_t cnt_off, keys_off, part_off, total;
};

// One phase: `count` matrices of n x k that read the same staged
// activations (units and groups as in Geometry).
struct Phase {
  const uint8_t *w[kMaxGroup];
  float *logits[kMaxGroup];  // entries may be null in verify mode
  const uint8_t *staged;
  // 32-bit: a matrix is smaller than 4 GiB, so n, its row bytes, its tiles
  // and its units (fewer than 2^31) all fit
  int n, row_bytes;
  int n_tiles;  // ceil(n / 16)
  int units;
  int count, kb, n_wg_per, n_groups;
};

struct GemvLaunch {
  Phase ph;            // single launches: the launch's phase
  const Phase *chain;  // chain launches: device table of n_phases phases (else null)
  int n_phases;
  unsigned *bar;       // chain: barrier count (scratch + kBarOff)
  unsigned *err;       // chain: time-out flag (scratch + kErrOff)
  unsigned *epoch;     // chain: launch epoch (scratch + kEpochOff)
  unsigned long long *flags;  // chain: per-workgroup release flags, 256 bytes apart
  int m;
  int layout;       // KQ_LAYOUT_* (the weight format and its layout)
  float *partials;
  unsigned *done;
  unsigned *group_cnt;
  unsigned long long *wg_keys;
  int32_t *argmax_out;  // verify only: row m's argmax at argmax_out[m - argmax_from], m >= argmax_from
  int argmax_from;
  int32_t *head_out;    // verify only, may be null: row 0's argmax
  int32_t *accept_out;  // verify only, may be null (then no accept decision)
  int32_t draft[kMaxTreeRows];   // linear: draft[i] judged by row i; tree: token of node i (i >= 1)
  int32_t parent[kMaxTreeRows];  // tree: parent of node i (i >= 1)
  int k_draft;                   // linear drafts (0: no linear accept)
  const int32_t *draft_dev;      // linear, may be null: the k_draft tokens in device memory (else draft[])
  int tree;                      // 1: tree accept over m nodes
  int32_t *path_out;             // tree, may be null: the accepted path's nodes
  int verify;
  // Staged activations of a single launch: block b's record at b * x_rec
  // (x_rec = the staged slices per block times kStageBytes).
  unsigned x_rec;
  // single launches (no chain table): 1 runs the launch's one phase on
  // kq_chain_kernel (plain Q4_K products of the 128-row geometry, m <= 16),
  // with kq_gemv_kernel's last-arrival reduction of split row groups
  int chain_single;
  Geometry g;
};

Geometry geometry(int64_t n, int64_t k, int count, int fmt = kFmtQ4, int ms = 1);
// the one scratch layout of every call on `count` matrices of n x k
ScratchLayout scratch_layout(int64_t n, int64_t k, int count, int max_ms);

// Kernel launches (return a hipError_t as int).
// kq_stage_kernel also zeroes the control words of `ctrl` (a scratch area
// laid out as above for n_groups row groups) when ctrl is not null.
int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *ctrl, int64_t n_groups,
                 void *stream);  // row_slices(m) records per block
int launch_gemv(const GemvLaunch &a, void *stream);
// Workgroups of the chain kernel (8 waves of one 16-row tile) the current
// device holds at once, or a negative HIP error code.
int chain_capacity();
int launch_fill(unsigned *p, int64_t n_words, void *stream, unsigned value = 0u);
// Copy one 32-bit device word to the host on `stream` and wait for the
// stream (a hipError_t as int).
int read_device_word(const unsigned *dev, unsigned *host, void *stream);
// Device address of the current device's copy of the library's fixed
// workspace (KQ_NOALLOC_MAX_BYTES, 256-byte aligned), looked up once per
// device (a hipError_t as int).
int noalloc_workspace(void **ptr);
int launch_tile(const uint8_t *w, int64_t n, int64_t k, uint8_t *out, void *stream, int fmt = kFmtQ4);
int launch_stream_probe(const uint8_t *p, int64_t chunks, unsigned *sink, int blocks, void *stream);
// Softmax rows: chunks of a row (4,096 logits each) and the two-pass launch
// (part: rows x chunks float pairs of workspace).
int softmax_chunks(int64_t n);
// out[i] = rows[i][tokens[i]], i < count (NaN for a token outside [0, n))
int launch_gather(const float *rows, int64_t n, const int32_t *tokens, int count, float *out, void *stream);
int launch_softmax(const float *logits, int m, int64_t n, float temperature, float cap, float *part, float *probs,
                   void *stream);

}  // namespace kq
