// kq_internal.h -- layout constants and launch entry points shared by the
// C-ABI wrapper (kq_api.cpp) and the HIP kernels (kq_kernels.hip).
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace kq {

constexpr int64_t kQK = 256;          // weights per Q4_K super-block
constexpr int64_t kBlockBytes = 144;  // bytes per super-block
constexpr int kMaxRows = 16;          // verify rows per call (block size of the draft)
constexpr int kMaxGroup = 8;          // matrices per grouped launch

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

// Scratch area of the main kernel:
//   [0, 256)      done counter (u32) at 0                    -- zero between calls
//   cnt_off       per-workgroup-column split-K arrivals (u32) -- zero between calls
//   keys_off      per-workgroup-column argmax keys [n_wg][16] (u64)
//   part_off      split-K partial sums [splits][count][16][n] fp32

struct Geometry {
  int count;     // matrices in the launch (same n, k, activations)
  int waves;     // waves per workgroup (4 or 8)
  int tpw;       // 16-row tiles per wave (1, 2 or 4)
  int n_wg_per;  // workgroup columns per matrix (16 * tpw * waves rows each)
  int n_wg;      // workgroup columns in total = count * n_wg_per
  int splits;    // workgroups along k
  int qps;       // quads per split
  int quads;     // total quads
};

struct ScratchLayout {
  size_t cnt_off, keys_off, part_off, ctrl_bytes, total;
};

struct GemvLaunch {
  const uint8_t *w[kMaxGroup];
  float *logits[kMaxGroup];  // entries may be null in verify mode
  int64_t n, k, row_bytes;
  int m;
  const uint8_t *staged;
  float *partials;
  unsigned *done;
  unsigned *tile_cnt;
  unsigned long long *wg_keys;
  int32_t *argmax_out;  // verify only
  int32_t *accept_out;  // verify only
  int32_t draft[kMaxRows];
  int k_draft;
  int verify;
  Geometry g;
};

Geometry geometry(int64_t n, int64_t k, int count);
ScratchLayout scratch_layout(int64_t n, int64_t k, int count);

// Kernel launches (return a hipError_t as int).
int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *zero_words,
                 int64_t n_zero_words, void *stream);
int launch_gemv(const GemvLaunch &a, void *stream);
int launch_fill(unsigned *p, int64_t n_words, void *stream);

}  // namespace kq
