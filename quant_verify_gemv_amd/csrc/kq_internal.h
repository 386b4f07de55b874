// kq_internal.h -- layout constants and launch entry points shared by the
// C-ABI wrapper (kq_api.cpp) and the HIP kernels (kq_kernels.hip).
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace kq {

constexpr int64_t kQK = 256;          // weights per Q4_K super-block
constexpr int64_t kBlockBytes = 144;  // bytes per super-block
constexpr int kMaxRows = 16;          // verify rows per call (block size of the draft)
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;

// Activations are staged in "quads" of 4 super-blocks (1,024 columns) that
// share one power-of-two scale per row. Per quad:
//   XA [4 blocks][8 k-steps][hi,lo][64 lanes][8 x fp16]   65,536 B
//   XS [hi,lo][64 lanes][8 x fp16]  (sub-block sums)         2,048 B
//   XI [16] fp32 (per-row 2^-e)                                 64 B
constexpr int64_t kQuadK = 1024;
constexpr int64_t kXaBlockBytes = 16384;
constexpr int64_t kXsOffset = 65536;
constexpr int64_t kXiOffset = 65536 + 2048;
constexpr int64_t kQuadBytes = 67840;  // 67,648 rounded up to 256

// Control words at the start of a scratch area (all zero between calls).
//   [0, 256)      done counter (u32) at 0
//   [256, ...)    per-workgroup-column split-K arrival counters (u32)
//   then          per-workgroup-column argmax keys [n_wg][16] (u64)
//   then          split-K partial sums [splits][16][n] fp32 (not control)

struct Geometry {
  int nt;       // 16-row tiles per wave
  int n_wg;     // workgroups along n
  int splits;   // workgroups along k
  int qps;      // quads per split
  int quads;    // total quads
};

struct ScratchLayout {
  size_t cnt_off, keys_off, part_off, ctrl_bytes, total;
};

struct GemvLaunch {
  const uint8_t *w;
  int64_t n, k, row_bytes;
  int m;
  const uint8_t *staged;
  float *logits;        // may be null in verify mode
  float *partials;      // [splits][16][n]
  unsigned *done;
  unsigned *tile_cnt;   // [n_wg]
  unsigned long long *wg_keys;  // [n_wg][16]
  int32_t *argmax_out;  // verify only
  int32_t *accept_out;  // verify only
  int32_t draft[kMaxRows];
  int k_draft;
  int verify;
  Geometry g;
};

Geometry geometry(int64_t n, int64_t k);
ScratchLayout scratch_layout(int64_t n, int64_t k);

// Kernel launches (return a hipError_t as int).
int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *zero_words,
                 int64_t n_zero_words, void *stream);
int launch_gemv(const GemvLaunch &a, void *stream);
int launch_fill(unsigned *p, int64_t n_words, void *stream);

}  // namespace kq
