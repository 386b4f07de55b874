// kq_api.cpp -- the C ABI declared in include/kq.h: argument validation
// (always before any HIP call), workspace layout, launch geometry.
#include "kq.h"

#include <math.h>
#include <stdint.h>
#include <string.h>


#include "kq_internal.h"

namespace kq {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The kernels address a weight matrix (either layout, rows rounded up to a
// 16-row tile) and a staged activation block with 32-bit offsets, so both
// must be smaller than 4 GiB.
static bool shape_ok(int64_t n, int64_t k, int fmt = kFmtQ4) {
  if (!(n >= 1 && n < ((int64_t)1 << 31) && k > 0 && k % kQK == 0 && k <= ((int64_t)1 << 28))) return false;
  const int64_t kb = k / kQK;
  const int64_t limit = (int64_t)1 << 32;
  return cdiv(n, 16) * 16 * kb * fmt_block_bytes(fmt) < limit && kb * kStageBytes < limit;
}

// Launch geometry: persistent workgroups, one per CU (their LDS activation
// ring of 8 blocks fills most of a CU's 160 KB), each taking an equal,
// contiguous run of (row group, block) units. Row groups are 256 rows (8
// waves of two 16-row tiles) for 131,072 rows or more (the LM head), 192
// rows (12 waves, three per SIMD, one tile each) from 32,768 rows (gate and
// up together), and 128 rows (8 waves, one tile each) below that, where a
// taller group would leave too few groups to share among 256 workgroups.
// Barriers every 4 units. Measured on MI355X with the shapes of the 52-layer
// stack, the DFlash fc projection and the LM head.
static constexpr int64_t kCUs = 256;

struct Shape {
  int waves, tpw, per_cu, bi, depth;
};

static Shape pick_shape(int64_t n, int count, int fmt, int ms) {
#ifdef KQ_GEOM_WAVES  // build-time override for tuning sweeps
#ifndef KQ_GEOM_BI
#define KQ_GEOM_BI 1
#endif
#ifndef KQ_GEOM_DEPTH
#define KQ_GEOM_DEPTH 4
#endif
  (void)n;
  (void)count;
  (void)fmt;
  (void)ms;
  return {KQ_GEOM_WAVES, KQ_GEOM_TPW, KQ_GEOM_PER_CU, KQ_GEOM_BI, KQ_GEOM_DEPTH};
#endif
  const int64_t rows = n * count;
  // Two activation slices (17 to 32 rows): the LDS ring shrinks to 4
  // blocks (every block now holds 2 staged slices) so that it still fits a
  // CU's LDS, with three weight register sets and two tiles per wave (each
  // activation read from LDS feeds 32 weight rows: 20 % faster than one
  // tile on the LM head). Three or four slices (33 to 64 rows): the ring
  // holds two blocks of 3 or 4 slices (101,760 or 135,680 bytes), two
  // weight register sets, two tiles per wave; every format.
  if (ms >= 3) return Shape{8, 2, 1, 1, 2};
  if (ms > 1) return Shape{8, 2, 1, 2, 3};
  // Q5_K and Q6_K (two more registers per tile and register set): two
  // tiles per wave from 131,072 rows (7-9 % faster than 12 one-tile waves on
  // the LM head), 12 waves of one tile from 32,768 rows, else 8
  if (fmt != kFmtQ4)
    return rows >= 131072 ? Shape{8, 2, 1, 4, 4} : rows >= 32768 ? Shape{12, 1, 1, 4, 4} : Shape{8, 1, 1, 4, 4};
  if (rows >= 131072) return {8, 2, 1, 4, 4};
  if (rows >= 32768) return {12, 1, 1, 4, 4};
  return {8, 1, 1, 4, 4};
}

Geometry geometry(int64_t n, int64_t k, int count, int fmt, int ms) {
  Geometry g;
  const Shape sh = pick_shape(n, count, fmt, ms);
  g.ms = ms;
  g.count = count;
  g.waves = sh.waves;
  g.tpw = sh.tpw;
  g.bi = sh.bi;
  g.depth = sh.depth;
  g.rows = 16 * sh.waves * sh.tpw;
  g.n_wg_per = (int)cdiv(n, g.rows);
  g.n_groups = g.count * g.n_wg_per;
  g.kb = (int)(k / kQK);
  g.units = (int64_t)g.n_groups * g.kb;
  // persistent workgroups: as many as the CUs hold at once
  int64_t slots = kCUs * sh.per_cu;
#ifdef KQ_GEOM_SPLIT  // build-time override for tuning sweeps: row groups x splits workgroups
  slots = (int64_t)g.n_groups * KQ_GEOM_SPLIT;
#endif
  g.n_wg = (int)(g.units < slots ? g.units : slots);
  return g;
}

// One layout for every call on `count` matrices of n x k, whatever the
// weight format and the launch's slice count: the arrival counters cover the
// most row groups and the keys the most workgroups of any of these
// geometries, and the partials come last. The offsets then never depend on
// the call, so a scratch shared by calls of different row counts or formats
// never has one launch's argmax keys or partials where another expects its
// zeroed counters. The partials cover
// the largest size of the launches of calls of up to max_ms slices (16
// max_ms rows); a call of fewer rows needs only that much.
ScratchLayout scratch_layout(int64_t n, int64_t k, int count, int max_ms) {
  size_t groups = 0, wgs = 0, part = 0;
  for (int f = kFmtQ4; f <= kFmtQ6; ++f) {
    if (!shape_ok(n, k, f)) continue;
    for (int ms = 1; ms <= 4; ++ms) {
      const Geometry g = geometry(n, k, count, f, ms);
      const size_t pb = sizeof(float) * (size_t)g.n_wg * 2 * kMaxRows * ms * (size_t)g.rows;
      groups = (size_t)g.n_groups > groups ? (size_t)g.n_groups : groups;
      wgs = (size_t)g.n_wg > wgs ? (size_t)g.n_wg : wgs;
      if (ms <= max_ms) part = pb > part ? pb : part;
    }
  }
  ScratchLayout s;
  s.cnt_off = kCntOff;
  s.keys_off = align256(s.cnt_off + sizeof(unsigned) * kCntStride * groups);
  s.part_off = align256(s.keys_off + sizeof(unsigned long long) * kMaxTreeRows * wgs);
  s.total = s.part_off + align256(part);
  return s;
}

// The staged records of k columns for m rows stay below 4 GiB (32-bit
// offsets).
static bool staged_ok(int64_t k, int m) {
  return k > 0 && k % kQK == 0 && k <= ((int64_t)1 << 28) && m >= 1 && m <= kMaxTreeRows &&
         (k / kQK) * row_slices(m) * kStageBytes < ((int64_t)1 << 32);
}

}  // namespace kq

using namespace kq;

extern "C" {

const char *kq_status_string(kq_status s) {
  switch (s) {
    case KQ_OK: return "KQ_OK";
    case KQ_ERR_NULL: return "KQ_ERR_NULL: a required pointer is NULL";
    case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE: m, n or k out of range";
    case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN: misaligned pointer";
    case KQ_ERR_TOKEN: return "KQ_ERR_TOKEN: draft token outside [0, n)";
    case KQ_ERR_WORKSPACE: return "KQ_ERR_WORKSPACE: workspace too small";
    case KQ_ERR_LAUNCH: return "KQ_ERR_LAUNCH: HIP launch failed";
    default: return "KQ_ERR_UNKNOWN";
  }
}

size_t kq_staged_bytes(int64_t k) { return kq_staged_bytes_rows(k, kMaxRows); }

size_t kq_staged_bytes_rows(int64_t k, int m) {
  if (!staged_ok(k, m)) return 0;
  return (size_t)(k / kQK) * (size_t)row_slices(m) * (size_t)kStageBytes;
}

// Scratch for `count` matrices: the one layout of every format and slice
// count.
static size_t scratch_any_fmt(int64_t n, int64_t k, int count) {
  return scratch_layout(n, k, count, row_slices(kMaxTreeRows)).total;
}

size_t kq_scratch_bytes(int64_t n, int64_t k) {
  if (!shape_ok(n, k)) return 0;
  return scratch_any_fmt(n, k, 1);
}

size_t kq_group_scratch_bytes(int64_t n, int64_t k, int count) {
  if (!shape_ok(n, k) || count < 1 || count > kMaxGroup) return 0;
  return scratch_any_fmt(n, k, count);
}

size_t kq_workspace_bytes(int64_t n, int64_t k, int m) {
  if (!shape_ok(n, k) || !staged_ok(k, m)) return 0;
  return align256(kq_staged_bytes_rows(k, m)) + scratch_layout(n, k, 1, row_slices(m)).total;
}

kq_status kq_launch_geometry(int64_t n, int64_t k, int *waves, int *tiles_per_wave,
                             int *workgroups, int64_t *units) {
  if (!shape_ok(n, k)) return KQ_ERR_SHAPE;
  const Geometry g = geometry(n, k, 1);
  if (waves) *waves = g.waves;
  if (tiles_per_wave) *tiles_per_wave = g.tpw;
  if (workgroups) *workgroups = g.n_wg;
  if (units) *units = g.units;
  return KQ_OK;
}

static inline bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t kq_tiled_bytes(int64_t n, int64_t k) { return kq_tiled_bytes_fmt(KQ_LAYOUT_TILED16, n, k); }

size_t kq_tiled_bytes_fmt(int layout, int64_t n, int64_t k) {
  if (layout == KQ_LAYOUT_ROWS || layout_fmt(layout) < 0 || !shape_ok(n, k, layout_fmt(layout))) return 0;
  return (size_t)cdiv(n, 16) * (size_t)(k / kQK) * 16 * (size_t)fmt_block_bytes(layout_fmt(layout));
}

kq_status kq_tile_weights(const void *w_q4k, int64_t n, int64_t k, void *w_tiled, size_t tiled_bytes,
                          void *stream) {
  return kq_tile_weights_fmt(KQ_LAYOUT_TILED16, w_q4k, n, k, w_tiled, tiled_bytes, stream);
}

kq_status kq_tile_weights_fmt(int layout, const void *w_rows, int64_t n, int64_t k, void *w_tiled,
                              size_t tiled_bytes, void *stream) {
  if (!w_rows || !w_tiled) return KQ_ERR_NULL;
  const int fmt = layout_fmt(layout);
  if (layout == KQ_LAYOUT_ROWS || fmt < 0 || !shape_ok(n, k, fmt)) return KQ_ERR_SHAPE;
  if (!al(w_rows, fmt == kFmtQ6 ? 2 : 16) || !al(w_tiled, 16)) return KQ_ERR_ALIGN;
  const size_t need = kq_tiled_bytes_fmt(layout, n, k);
  if (tiled_bytes < need) return KQ_ERR_WORKSPACE;
  const uintptr_t a0 = (uintptr_t)w_rows, a1 = a0 + (uintptr_t)(n * (k / kQK) * fmt_block_bytes(fmt));
  const uintptr_t b0 = (uintptr_t)w_tiled, b1 = b0 + (uintptr_t)need;
  if (a0 < b1 && b0 < a1) return KQ_ERR_SHAPE;  // buffers overlap
  if (launch_tile((const uint8_t *)w_rows, n, k, (uint8_t *)w_tiled, stream, fmt)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_workspace_init(void *workspace, size_t bytes, void *stream) {
  if (!workspace) return KQ_ERR_NULL;
  if (!al(workspace, 256)) return KQ_ERR_ALIGN;
  if (bytes < 256) return KQ_ERR_WORKSPACE;
  if (launch_fill((unsigned *)workspace, (int64_t)(bytes / 4), stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_stage_rows(const float *x, int m, int64_t k, void *staged, size_t staged_bytes,
                        void *stream) {
  if (!x || !staged) return KQ_ERR_NULL;
  if (!staged_ok(k, m)) return KQ_ERR_SHAPE;
  if (!al(x, 16) || !al(staged, 256)) return KQ_ERR_ALIGN;
  if (staged_bytes < kq_staged_bytes_rows(k, m)) return KQ_ERR_WORKSPACE;
  if (launch_stage(x, m, k, (uint8_t *)staged, nullptr, 0, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

// The kernel's description of one phase: count matrices of n x k on one
// staged activation block, cut into units by geometry g.
static void fill_phase(Phase &ph, const Geometry &g, const void *const *w, float *const *logits, int count,
                       int64_t n, int64_t k, const void *staged) {
  memset(&ph, 0, sizeof(ph));
  for (int i = 0; i < count; ++i) {
    ph.w[i] = (const uint8_t *)w[i];
    ph.logits[i] = logits ? logits[i] : nullptr;
  }
  ph.staged = (const uint8_t *)staged;
  ph.n = (int)n;
  ph.row_bytes = (int)((k / kQK) * kBlockBytes);
  ph.n_tiles = (int)cdiv(n, 16);
  ph.units = (int)g.units;
  ph.count = count;
  ph.kb = g.kb;
  ph.n_wg_per = g.n_wg_per;
  ph.n_groups = g.n_groups;
}

// Shared validation + launch of the main kernel on staged activations for
// `count` matrices of the same shape (verify: count == 1).
// verify: per-row argmax, written from row argmax_from on (0 for the verify
// step, 1 for a draft block's proposals), row 0's also to head_out when not
// null, and the accept decision against draft_host when accept_out is not
// null.
static kq_status run(const void *const *w, int layout, int count, int64_t n, int64_t k,
                     const void *staged, int m, float *const *logits, bool verify,
                     const int32_t *draft_host, int32_t *argmax, int32_t *accept_out, int argmax_from,
                     int32_t *head_out, void *scratch, size_t scratch_bytes, const float *x_to_stage,
                     void *stream, const int32_t *tree_parent = nullptr, int32_t *path_out = nullptr,
                     const int32_t *draft_dev = nullptr, bool dry = false) {
  if (!w || !staged || !scratch) return KQ_ERR_NULL;
  const int fmt = layout_fmt(layout);
  if (fmt < 0) return KQ_ERR_SHAPE;
  if (count < 1 || count > kMaxGroup || (verify && count != 1)) return KQ_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    if (!w[i]) return KQ_ERR_NULL;
    if (!verify && (!logits || !logits[i])) return KQ_ERR_NULL;
  }
  if (verify && (!argmax || (!accept_out && argmax_from == 0))) return KQ_ERR_NULL;
  if (verify && accept_out && m > 1 && !draft_host && !draft_dev) return KQ_ERR_NULL;
  if (!shape_ok(n, k, fmt) || !staged_ok(k, m)) return KQ_ERR_SHAPE;
  for (int i = 0; i < count; ++i)
    if (!al(w[i], 16)) return KQ_ERR_ALIGN;
  if (!al(staged, 256) || !al(scratch, 256)) return KQ_ERR_ALIGN;
  if (x_to_stage && !al(x_to_stage, 16)) return KQ_ERR_ALIGN;
  // staged slices: the launch runs all of them in one pass over the weights
  const int ms = row_slices(m);
  const ScratchLayout sl = scratch_layout(n, k, count, ms);
  if (scratch_bytes < sl.total) return KQ_ERR_WORKSPACE;
  GemvLaunch a;
  memset(&a, 0, sizeof(a));
  if (verify && accept_out && tree_parent) {
    // node 0 is the root; every other node names an earlier node as parent
    if (tree_parent[0] != -1) return KQ_ERR_SHAPE;
    for (int i = 1; i < m; ++i)
      if (tree_parent[i] < 0 || tree_parent[i] >= i) return KQ_ERR_SHAPE;
    for (int i = 1; i < m; ++i) {
      if (draft_host[i] < 0 || (int64_t)draft_host[i] >= n) return KQ_ERR_TOKEN;
      a.draft[i] = draft_host[i];
      a.parent[i] = tree_parent[i];
    }
    a.parent[0] = -1;
    a.tree = 1;
    a.path_out = path_out;
  } else if (verify && accept_out && draft_dev) {
    if (m > 1 && !al(draft_dev, 4)) return KQ_ERR_ALIGN;
    a.draft_dev = draft_dev;  // read by the kernel; not validated on the host
  } else if (verify && accept_out) {
    for (int i = 0; i < m - 1; ++i) {
      if (draft_host[i] < 0 || (int64_t)draft_host[i] >= n) return KQ_ERR_TOKEN;
      a.draft[i] = draft_host[i];
    }
  }
  a.layout = layout;
  a.argmax_out = argmax;
  a.argmax_from = argmax_from;
  a.head_out = head_out;
  a.accept_out = accept_out;
  a.k_draft = verify && accept_out && !tree_parent ? m - 1 : 0;
  a.verify = verify ? 1 : 0;
  a.x_rec = (unsigned)(ms * kStageBytes);
  uint8_t *sc = (uint8_t *)scratch;
  a.g = geometry(n, k, count, fmt, ms);
  fill_phase(a.ph, a.g, w, logits, count, n, k, staged);
  a.done = (unsigned *)sc;
  a.group_cnt = (unsigned *)(sc + sl.cnt_off);
  a.wg_keys = (unsigned long long *)(sc + sl.keys_off);
  a.partials = (float *)(sc + sl.part_off);
  a.m = m;
  // 17 to 64 rows: one pass over the weights at two to four slices, on
  // two-tile waves (each activation read from LDS feeds 32 weight rows). At
  // 33 to 64 rows it took 18-25 % less time than two passes (rows 0-31,
  // then the rest) on the 131,072-row LM head (40 to 64 tree nodes; Q4_K,
  // Q5_K and Q6_K, MI355X, interleaved).
  //
  // Plain Q4_K products of the 128-row geometry (at most 16 rows) run on
  // the chain kernel's specialised waves as a one-phase launch (its own
  // last-arrival reduction, so no co-residency is needed): same units and
  // summation orders, so the results are bitwise those of kq_gemv_kernel;
  // measured 2-3 % faster on the 33,280 -> 6,656 fc and about 5 % on
  // 6,656 x 6,656 (MI355X, interleaved graphs of back-to-back calls).
  if (!verify && fmt == kFmtQ4 && ms == 1 && a.g.waves * a.g.tpw * 16 == kChainRows) {
    a.chain_single = 1;
    a.bar = (unsigned *)(sc + kBarOff);
    a.err = (unsigned *)(sc + kErrOff);
    a.epoch = (unsigned *)(sc + kEpochOff);
  }
  if (dry) return KQ_OK;  // every check passed; nothing enqueued
  if (x_to_stage) {
    if (launch_stage(x_to_stage, m, k, (uint8_t *)staged, (unsigned *)scratch, a.g.n_groups, stream))
      return KQ_ERR_LAUNCH;
  }
  if (launch_gemv(a, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_gemv_staged(const void *w_q4k, int layout, int64_t n, int64_t k, const void *staged, int m,
                         float *logits, void *scratch, size_t scratch_bytes, void *stream) {
  return run(&w_q4k, layout, 1, n, k, staged, m, &logits, false, nullptr, nullptr, nullptr, 0, nullptr, scratch,
             scratch_bytes, nullptr, stream);
}

kq_status kq_gemv_staged_group(const void *const *w_q4k, int layout, int count, int64_t n, int64_t k,
                               const void *staged, int m, float *const *logits, void *scratch,
                               size_t scratch_bytes, void *stream) {
  if (!w_q4k || !logits) return KQ_ERR_NULL;
  return run(w_q4k, layout, count, n, k, staged, m, logits, false, nullptr, nullptr, nullptr, 0, nullptr, scratch,
             scratch_bytes, nullptr, stream);
}

kq_status kq_verify_staged(const void *w_q4k, int layout, int64_t n, int64_t k, const void *staged, int m,
                           const int32_t *draft_host, int32_t *argmax, int32_t *accept_out,
                           float *logits_or_null, void *scratch, size_t scratch_bytes,
                           void *stream) {
  return run(&w_q4k, layout, 1, n, k, staged, m, &logits_or_null, true, draft_host, argmax, accept_out, 0,
             nullptr, scratch, scratch_bytes, nullptr, stream);
}

kq_status kq_verify_staged_dev(const void *w, int layout, int64_t n, int64_t k, const void *staged, int m,
                               const int32_t *draft_dev, int32_t *argmax, int32_t *accept_out,
                               float *logits_or_null, void *scratch, size_t scratch_bytes, void *stream) {
  if (!argmax || !accept_out) return KQ_ERR_NULL;
  if (m > 1 && !draft_dev) return KQ_ERR_NULL;
  return run(&w, layout, 1, n, k, staged, m, &logits_or_null, true, nullptr, argmax, accept_out, 0, nullptr,
             scratch, scratch_bytes, nullptr, stream, nullptr, nullptr, draft_dev);
}

kq_status kq_verify_tree_staged(const void *w, int layout, int64_t n, int64_t k, const void *staged, int m,
                                const int32_t *parent_host, const int32_t *token_host, int32_t *argmax,
                                int32_t *accept_out, int32_t *path_out_or_null, float *logits_or_null,
                                void *scratch, size_t scratch_bytes, void *stream) {
  if (!parent_host || !token_host || !argmax || !accept_out) return KQ_ERR_NULL;
  return run(&w, layout, 1, n, k, staged, m, &logits_or_null, true, token_host, argmax, accept_out, 0, nullptr,
             scratch, scratch_bytes, nullptr, stream, parent_host, path_out_or_null);
}

static kq_status split_workspace(int64_t n, int64_t k, int m, void *ws, size_t ws_bytes,
                                 void **staged, void **scratch, size_t *scratch_bytes) {
  if (!ws) return KQ_ERR_NULL;
  if (!shape_ok(n, k) || !staged_ok(k, m)) return KQ_ERR_SHAPE;
  if (!al(ws, 256)) return KQ_ERR_ALIGN;
  const size_t need = kq_workspace_bytes(n, k, m);
  if (ws_bytes < need) return KQ_ERR_WORKSPACE;
  const size_t st = align256(kq_staged_bytes_rows(k, m));
  *staged = ws;
  *scratch = (uint8_t *)ws + st;
  *scratch_bytes = ws_bytes - st;
  return KQ_OK;
}

kq_status kq_gemv_rows(const void *w_q4k, int64_t n, int64_t k, const float *x, int m,
                       float *logits, void *workspace, size_t workspace_bytes, void *stream) {
  if (!w_q4k || !x || !logits) return KQ_ERR_NULL;
  void *staged, *scratch;
  size_t sb;
  kq_status s = split_workspace(n, k, m, workspace, workspace_bytes, &staged, &scratch, &sb);
  if (s != KQ_OK) return s;
  return run(&w_q4k, KQ_LAYOUT_ROWS, 1, n, k, staged, m, &logits, false, nullptr, nullptr, nullptr, 0,
             nullptr, scratch, sb, x, stream);
}

// kq_verify_argmax_accept; dry: every argument check, nothing enqueued
static kq_status verify_rows(const void *w_q4k, int64_t n, int64_t k, const float *x, int m,
                             const int32_t *draft_host, int32_t *argmax, int32_t *accept_out,
                             float *logits_or_null, void *workspace, size_t workspace_bytes, void *stream,
                             bool dry) {
  if (!w_q4k || !x || !argmax || !accept_out) return KQ_ERR_NULL;
  if (m > 1 && !draft_host) return KQ_ERR_NULL;
  void *staged, *scratch;
  size_t sb;
  kq_status s = split_workspace(n, k, m, workspace, workspace_bytes, &staged, &scratch, &sb);
  if (s != KQ_OK) return s;
  return run(&w_q4k, KQ_LAYOUT_ROWS, 1, n, k, staged, m, &logits_or_null, true, draft_host, argmax,
             accept_out, 0, nullptr, scratch, sb, x, stream, nullptr, nullptr, nullptr, dry);
}

kq_status kq_verify_argmax_accept(const void *w_q4k, int64_t n, int64_t k, const float *x, int m,
                                  const int32_t *draft_host, int32_t *argmax, int32_t *accept_out,
                                  float *logits_or_null, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  return verify_rows(w_q4k, n, k, x, m, draft_host, argmax, accept_out, logits_or_null, workspace,
                     workspace_bytes, stream, false);
}

kq_status kq_verify_argmax_accept_noalloc(const void *w_q4k, int64_t n, int64_t k, const float *x, int m,
                                          const int32_t *draft_host, int32_t *argmax, int32_t *accept_out,
                                          float *logits_or_null, void *stream) {
  if (!w_q4k || !x || !argmax || !accept_out) return KQ_ERR_NULL;
  if (m > 1 && !draft_host) return KQ_ERR_NULL;
  const size_t need = kq_workspace_bytes(n, k, m);
  if (!need) return KQ_ERR_SHAPE;
  if (need > (size_t)KQ_NOALLOC_MAX_BYTES) return KQ_ERR_WORKSPACE;
  // every argument check of the call below, on a stand-in workspace address
  // (256-byte aligned, never used), so that a refused call makes no HIP call
  kq_status s = verify_rows(w_q4k, n, k, x, m, draft_host, argmax, accept_out, logits_or_null,
                            (void *)(uintptr_t)256, need, stream, true);
  if (s != KQ_OK) return s;
  void *ws = nullptr;
  if (noalloc_workspace(&ws) || !ws) return KQ_ERR_LAUNCH;
  return kq_verify_argmax_accept(w_q4k, n, k, x, m, draft_host, argmax, accept_out, logits_or_null, ws, need,
                                 stream);
}

size_t kq_stream_probe_sink_bytes(void) { return 4 * 8192; }

kq_status kq_stream_probe(const void *buf, size_t bytes, uint32_t *sink, size_t sink_bytes, void *stream) {
  if (!buf || !sink) return KQ_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return KQ_ERR_SHAPE;
  if (!al(buf, 16) || !al(sink, 4)) return KQ_ERR_ALIGN;
  const int blocks = 8192;  // 32 contiguous slabs per CU
  if (sink_bytes < (size_t)4 * blocks) return KQ_ERR_WORKSPACE;
  if (launch_stream_probe((const uint8_t *)buf, (int64_t)(bytes / 16), sink, blocks, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

size_t kq_chain_table_bytes(int n_phases) {
  if (n_phases < 1 || n_phases > KQ_MAX_CHAIN_PHASES) return 0;
  return (size_t)n_phases * sizeof(Phase);
}

// Chain geometry: row groups of kChainRows rows (kq_chain_kernel's compute
// waves of one 16-row tile each; `tpw` is 1).
static Geometry chain_geometry(int64_t n, int64_t k, int count, int tpw) {
  Geometry g;
  g.count = count;
  g.waves = kChainRows / 16;
  g.tpw = tpw;
  g.bi = 4;
  g.depth = 4;
  g.ms = 1;
  g.rows = kChainRows * tpw;
  g.n_wg_per = (int)cdiv(n, g.rows);
  g.n_groups = count * g.n_wg_per;
  g.kb = (int)(k / kQK);
  g.units = (int64_t)g.n_groups * g.kb;
  g.n_wg = 0;
  return g;
}

// Tiles per wave of a chain's phases: one (two-tile waves, 256-row groups,
// measured slower on the stack's shapes and need more registers than fit).
static int chain_tpw() { return 1; }

// Chain scratch: control words, group counters, partials, then one
// 256-byte line per workgroup for its barrier release flag.
static size_t chain_part_off(int max_groups) {
  return align256((size_t)kCntOff + sizeof(unsigned) * kCntStride * (size_t)max_groups);
}
static size_t chain_flag_off(int max_groups, int64_t wg, int tpw) {
  return chain_part_off(max_groups) + align256(sizeof(float) * (size_t)wg * 2 * kMaxRows * kChainRows * (size_t)tpw);
}
static size_t chain_flag_bytes(int64_t wg) { return (size_t)wg * 256; }

kq_status kq_chain_encode(const kq_chain_phase *phases, int n_phases, int m, int layout, void *table_host,
                          size_t table_bytes, kq_chain_plan *plan) {
  if (!phases || !table_host || !plan) return KQ_ERR_NULL;
  if (n_phases < 1 || n_phases > KQ_MAX_CHAIN_PHASES || m < 1 || m > kMaxRows) return KQ_ERR_SHAPE;
  if (layout != KQ_LAYOUT_ROWS && layout != KQ_LAYOUT_TILED16) return KQ_ERR_SHAPE;
  int64_t min_units = -1;
  int max_groups = 0;
  const int tpw = chain_tpw();
  for (int i = 0; i < n_phases; ++i) {
    const kq_chain_phase &q = phases[i];
    if (q.count < 1 || q.count > kMaxGroup || !shape_ok(q.n, q.k)) return KQ_ERR_SHAPE;
    if (!q.staged) return KQ_ERR_NULL;
    for (int j = 0; j < q.count; ++j)
      if (!q.w_q4k[j] || !q.logits[j]) return KQ_ERR_NULL;
    for (int j = 0; j < q.count; ++j)
      if (!al(q.w_q4k[j], 16) || !al(q.logits[j], 4)) return KQ_ERR_ALIGN;
    if (!al(q.staged, 256)) return KQ_ERR_ALIGN;
    const Geometry g = chain_geometry(q.n, q.k, q.count, tpw);
    if (min_units < 0 || g.units < min_units) min_units = g.units;
    if (g.n_groups > max_groups) max_groups = g.n_groups;
  }
  if (table_bytes < kq_chain_table_bytes(n_phases)) return KQ_ERR_WORKSPACE;
  const int cap = chain_capacity();
  if (cap <= 0) return KQ_ERR_LAUNCH;
  const int64_t wg = min_units < cap ? min_units : cap;
  Phase *tab = (Phase *)table_host;
  for (int i = 0; i < n_phases; ++i) {
    const kq_chain_phase &q = phases[i];
    fill_phase(tab[i], chain_geometry(q.n, q.k, q.count, tpw), q.w_q4k, q.logits, q.count, q.n, q.k, q.staged);
  }
  memset(plan, 0, sizeof(*plan));
  plan->n_phases = n_phases;
  plan->m = m;
  plan->layout = layout;
  plan->workgroups = (int32_t)wg;
  plan->max_groups = max_groups;
  plan->tiles_per_wave = tpw;
  plan->table_bytes = kq_chain_table_bytes(n_phases);
  plan->scratch_bytes = chain_flag_off(max_groups, wg, tpw) + chain_flag_bytes(wg);
  return KQ_OK;
}

// Scratch bytes a plan needs, or 0 if the plan is not one kq_chain_encode
// could have written.
static bool chain_plan_fields_ok(const kq_chain_plan *plan) {
  return !(plan->n_phases < 1 || plan->n_phases > KQ_MAX_CHAIN_PHASES || plan->m < 1 || plan->m > kMaxRows ||
           plan->workgroups < 1 || plan->max_groups < 1 || plan->tiles_per_wave != 1 ||
           (plan->layout != KQ_LAYOUT_ROWS && plan->layout != KQ_LAYOUT_TILED16));
}
static size_t chain_plan_scratch(const kq_chain_plan *plan) {
  const size_t need = chain_flag_off(plan->max_groups, plan->workgroups, plan->tiles_per_wave) +
                      chain_flag_bytes(plan->workgroups);
  return plan->scratch_bytes == need ? need : 0;
}

kq_status kq_chain_scratch_init(const kq_chain_plan *plan, void *scratch, size_t scratch_bytes, void *stream) {
  if (!plan || !scratch) return KQ_ERR_NULL;
  if (!chain_plan_fields_ok(plan)) return KQ_ERR_SHAPE;
  if (!al(scratch, 256)) return KQ_ERR_ALIGN;
  const size_t need = chain_plan_scratch(plan);
  if (!need) return KQ_ERR_SHAPE;  // not a plan kq_chain_encode wrote
  if (scratch_bytes < need) return KQ_ERR_WORKSPACE;
  uint8_t *sc = (uint8_t *)scratch;
  const size_t p0 = chain_part_off(plan->max_groups);
  const size_t p1 = chain_flag_off(plan->max_groups, plan->workgroups, plan->tiles_per_wave);
  if (launch_fill((unsigned *)sc, (int64_t)(p0 / 4), stream)) return KQ_ERR_LAUNCH;
  if (launch_fill((unsigned *)(sc + p0), (int64_t)((p1 - p0) / 4), stream, 0xFFFFFFFFu)) return KQ_ERR_LAUNCH;
  if (launch_fill((unsigned *)(sc + p1), (int64_t)((need - p1) / 4), stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_gemv_chain(const void *table_dev, const kq_chain_plan *plan, void *scratch, size_t scratch_bytes,
                        void *stream) {
  if (!table_dev || !plan || !scratch) return KQ_ERR_NULL;
  if (!chain_plan_fields_ok(plan)) return KQ_ERR_SHAPE;
  if (!al(table_dev, 16) || !al(scratch, 256)) return KQ_ERR_ALIGN;
  const size_t need = chain_plan_scratch(plan);
  if (!need) return KQ_ERR_SHAPE;  // not a plan kq_chain_encode wrote
  if (scratch_bytes < need) return KQ_ERR_WORKSPACE;
  GemvLaunch a;
  memset(&a, 0, sizeof(a));
  uint8_t *sc = (uint8_t *)scratch;
  a.chain = (const Phase *)table_dev;
  a.n_phases = plan->n_phases;
  a.bar = (unsigned *)(sc + kBarOff);
  a.err = (unsigned *)(sc + kErrOff);
  a.m = plan->m;
  a.layout = plan->layout;
  a.done = (unsigned *)sc;
  a.group_cnt = (unsigned *)(sc + kCntOff);
  a.partials = (float *)(sc + chain_part_off(plan->max_groups));
  a.epoch = (unsigned *)(sc + kEpochOff);
  a.flags = (unsigned long long *)(sc + chain_flag_off(plan->max_groups, plan->workgroups, plan->tiles_per_wave));
  a.g = chain_geometry(kChainRows, kQK, 1, plan->tiles_per_wave);
  a.g.n_wg = plan->workgroups;
  if (launch_gemv(a, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_chain_status(const kq_chain_plan *plan, const void *scratch, size_t scratch_bytes, void *stream) {
  if (!plan || !scratch) return KQ_ERR_NULL;
  if (!chain_plan_fields_ok(plan)) return KQ_ERR_SHAPE;
  if (!al(scratch, 256)) return KQ_ERR_ALIGN;
  const size_t need = chain_plan_scratch(plan);
  if (!need) return KQ_ERR_SHAPE;  // not a plan kq_chain_encode wrote
  if (scratch_bytes < need) return KQ_ERR_WORKSPACE;
  unsigned word = 0;
  if (read_device_word((const unsigned *)((const uint8_t *)scratch + kErrOff), &word, stream)) return KQ_ERR_LAUNCH;
  return word ? KQ_ERR_LAUNCH : KQ_OK;
}

size_t kq_softmax_workspace_bytes(int m, int64_t n) {
  if (m < 1 || m > 65535 || n < 1 || n >= ((int64_t)1 << 31)) return 0;
  return align256((size_t)m * (size_t)softmax_chunks(n) * 2 * sizeof(float));
}

kq_status kq_softmax_rows(const float *logits, int m, int64_t n, float temperature, float soft_cap, float *probs,
                          void *workspace, size_t workspace_bytes, void *stream) {
  if (!logits || !probs || !workspace) return KQ_ERR_NULL;
  if (m < 1 || m > 65535 || n < 1 || n >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
  if (!(temperature > 0.0f) || !isfinite(temperature) || !(soft_cap >= 0.0f) || !isfinite(soft_cap))
    return KQ_ERR_SHAPE;
  if (!al(logits, 4) || !al(probs, 4) || !al(workspace, 256)) return KQ_ERR_ALIGN;
  if (workspace_bytes < kq_softmax_workspace_bytes(m, n)) return KQ_ERR_WORKSPACE;
  if (launch_softmax(logits, m, n, temperature, soft_cap, (float *)workspace, probs, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

// Every token of one order row is in [0, n).
static bool order_row_ok(const int32_t *order, int64_t n) {
  for (int64_t j = 0; j < n; ++j)
    if (order[j] < 0 || (int64_t)order[j] >= n) return false;
  return true;
}

// Draw by walking `order`. A token's value is p[t], or, when q is given,
// max(p[t] - q[t], 0) / total; tokens whose value is not positive are skipped
// when `positive_only`. fp32 running sum, the first token whose sum exceeds
// u, else the last token walked; -1 when no token qualifies.
static int32_t sample_in_order(const float *p, const float *q, float total, const int32_t *order, int64_t n,
                               float u, bool positive_only) {
  float c = 0.0f;
  int32_t last = -1;
  for (int64_t j = 0; j < n; ++j) {
    const int32_t t = order[j];
    const float v = q ? fmaxf(p[t] - q[t], 0.0f) / total : p[t];
    if (positive_only && !(v > 0.0f)) continue;
    c = c + v;
    last = t;
    if (u < c) return t;
  }
  return last;
}

kq_status kq_gather_rows(const float *rows, int m, int64_t n, const int32_t *tokens, int count, float *out,
                         void *stream) {
  if (m < 1 || m > 65535 || n < 1 || n >= ((int64_t)1 << 31) || count < 0 || count > m) return KQ_ERR_SHAPE;
  if (count == 0) return KQ_OK;
  if (!rows || !tokens || !out) return KQ_ERR_NULL;
  if (!al(rows, 4) || !al(tokens, 4) || !al(out, 4)) return KQ_ERR_ALIGN;
  if (launch_gather(rows, n, tokens, count, out, stream)) return KQ_ERR_LAUNCH;
  return KQ_OK;
}

kq_status kq_speculative_first_reject(int k, const float *p_at, const float *q_at, const float *uniforms,
                                      int32_t *position) {
  if (!position || (k > 0 && (!p_at || !q_at || !uniforms))) return KQ_ERR_NULL;
  if (k < 0 || k >= kMaxRows) return KQ_ERR_SHAPE;
  // min(p / q, 1) that keeps a NaN ratio (fminf would return 1), so a NaN
  // (e.g. a gathered token outside the row) rejects
  int i = 0;
  for (; i < k; ++i) {
    const float r = p_at[i] / q_at[i];
    const float acceptance = q_at[i] <= 0.0f ? 1.0f : (r >= 1.0f ? 1.0f : r);
    if (!(uniforms[i] <= acceptance)) break;
  }
  *position = i;
  return KQ_OK;
}

kq_status kq_speculative_resample(int64_t n, const float *p_row, const float *q_row_or_null, const int32_t *order,
                                  float u, int32_t *token) {
  if (!p_row || !order || !token) return KQ_ERR_NULL;
  if (n < 1 || n >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
  if (!order_row_ok(order, n)) return KQ_ERR_TOKEN;
  int32_t t;
  if (q_row_or_null) {
    // the replacement comes from max(p - q, 0) divided by its sum (summed in
    // token order), or from p when that sum is not positive
    const float *q = q_row_or_null;
    float total = 0.0f;
    for (int64_t j = 0; j < n; ++j) total = total + fmaxf(p_row[j] - q[j], 0.0f);
    t = sample_in_order(p_row, total > 0.0f ? q : nullptr, total, order, n, u, true);
    if (t < 0) return KQ_ERR_SHAPE;  // a row without any positive probability
  } else {
    t = sample_in_order(p_row, nullptr, 0.0f, order, n, u, false);
  }
  *token = t;
  return KQ_OK;
}

kq_status kq_speculative_decide(int k, const int32_t *draft_tokens, int64_t n, const float *draft_rows,
                                const float *target_rows, const int32_t *orders, const float *uniforms,
                                int32_t *accepted, int32_t *next_token) {
  if (!target_rows || !orders || !uniforms || !accepted || !next_token) return KQ_ERR_NULL;
  if (k > 0 && (!draft_tokens || !draft_rows)) return KQ_ERR_NULL;
  if (k < 0 || k >= kMaxRows || n < 1 || n >= ((int64_t)1 << 31)) return KQ_ERR_SHAPE;
  for (int i = 0; i < k; ++i)
    if (draft_tokens[i] < 0 || (int64_t)draft_tokens[i] >= n) return KQ_ERR_TOKEN;
  float p_at[kMaxRows], q_at[kMaxRows];
  for (int i = 0; i < k; ++i) {
    p_at[i] = target_rows[(int64_t)i * n + draft_tokens[i]];
    q_at[i] = draft_rows[(int64_t)i * n + draft_tokens[i]];
  }
  int32_t j = 0, tok = 0;
  kq_status st = kq_speculative_first_reject(k, p_at, q_at, uniforms, &j);
  if (st != KQ_OK) return st;
  const float *p = target_rows + (int64_t)j * n;
  const int32_t *order = orders + (int64_t)j * n;
  st = j < k ? kq_speculative_resample(n, p, draft_rows + (int64_t)j * n, order, uniforms[j + 1], &tok)
             : kq_speculative_resample(n, p, nullptr, order, uniforms[k], &tok);
  if (st != KQ_OK) return st;
  *accepted = j;
  *next_token = tok;
  return KQ_OK;
}

// ---------------------------------------------------------------------------
// MT19937 (Matsumoto and Nishimura 1998): 624-word state, the twist
// x[k + 624] = x[k + 397] ^ ((x[k] & 0x80000000 | x[k + 1] & 0x7fffffff) A)
// with A the companion matrix of 0x9908b0df, and the tempering of each
// output word.
kq_status kq_mt19937_seed(kq_mt19937 *state, uint32_t seed) {
  if (!state) return KQ_ERR_NULL;
  state->mt[0] = seed;
  for (uint32_t i = 1; i < KQ_MT19937_WORDS; ++i) {
    const uint32_t prev = state->mt[i - 1];
    state->mt[i] = 1812433253u * (prev ^ (prev >> 30)) + i;
  }
  state->index = KQ_MT19937_WORDS;
  return KQ_OK;
}

static void mt_twist(kq_mt19937 *s) {
  constexpr int kN = KQ_MT19937_WORDS, kM = 397;
  for (int k = 0; k < kN; ++k) {
    const uint32_t y = (s->mt[k] & 0x80000000u) | (s->mt[(k + 1) % kN] & 0x7FFFFFFFu);
    s->mt[k] = s->mt[(k + kM) % kN] ^ (y >> 1) ^ ((y & 1u) ? 0x9908B0DFu : 0u);
  }
  s->index = 0;
}

static uint32_t mt_next(kq_mt19937 *s) {
  if (s->index >= KQ_MT19937_WORDS) mt_twist(s);
  uint32_t y = s->mt[s->index++];
  y ^= y >> 11;
  y ^= (y << 7) & 0x9D2C5680u;
  y ^= (y << 15) & 0xEFC60000u;
  y ^= y >> 18;
  return y;
}

static float mt_float(uint32_t w) { return (float)(w >> 8) * 0x1.0p-24f; }

kq_status kq_mt19937_u32(kq_mt19937 *state, uint32_t *out, int64_t count) {
  if (!state || (count > 0 && !out)) return KQ_ERR_NULL;
  if (count < 0 || state->index > KQ_MT19937_WORDS) return KQ_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) out[i] = mt_next(state);
  return KQ_OK;
}

kq_status kq_mt19937_uniform_f32(kq_mt19937 *state, float *out, int64_t count) {
  if (!state || (count > 0 && !out)) return KQ_ERR_NULL;
  if (count < 0 || state->index > KQ_MT19937_WORDS) return KQ_ERR_SHAPE;
  for (int64_t i = 0; i < count; ++i) out[i] = mt_float(mt_next(state));
  return KQ_OK;
}

kq_status kq_speculative_decide_mt(int k, const int32_t *draft_tokens, int64_t n, const float *draft_rows,
                                   const float *target_rows, const int32_t *orders, kq_mt19937 *rng,
                                   int32_t *accepted, int32_t *next_token) {
  // the outputs are checked here: the decision below writes to locals
  if (!rng || !accepted || !next_token) return KQ_ERR_NULL;
  if (rng->index > KQ_MT19937_WORDS) return KQ_ERR_SHAPE;
  if (k < 0 || k >= kMaxRows) return KQ_ERR_SHAPE;
  // the k + 1 draws any path can use, from a copy: position i reads draw i,
  // the token drawn after a rejection at i draw i + 1, the bonus draw k
  kq_mt19937 ahead = *rng;
  float u[kMaxRows + 1];
  for (int i = 0; i <= k; ++i) u[i] = mt_float(mt_next(&ahead));
  int32_t acc = 0, tok = 0;
  const kq_status st =
      kq_speculative_decide(k, draft_tokens, n, draft_rows, target_rows, orders, u, &acc, &tok);
  if (st != KQ_OK) return st;  // every check precedes the first draw: rng untouched
  const int used = acc < k ? acc + 2 : k + 1;
  for (int i = 0; i < used; ++i) (void)mt_next(rng);
  *accepted = acc;
  *next_token = tok;
  return KQ_OK;
}

static bool verify_length_ok(int length) { return length == 3 || length == 7 || length == 15; }

kq_status kq_draft_block_argmax(const void *w_q4k, int64_t n, int64_t k, const float *x, int verify_length,
                                int32_t *proposals, int32_t *head_or_null, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (!w_q4k || !x || !proposals) return KQ_ERR_NULL;
  if (!verify_length_ok(verify_length)) return KQ_ERR_SHAPE;
  const int m = verify_length + 1;
  void *staged, *scratch;
  size_t sb;
  kq_status s = split_workspace(n, k, m, workspace, workspace_bytes, &staged, &scratch, &sb);
  if (s != KQ_OK) return s;
  float *no_logits = nullptr;
  return run(&w_q4k, KQ_LAYOUT_ROWS, 1, n, k, staged, m, &no_logits, true, nullptr, proposals, nullptr, 1,
             head_or_null, scratch, sb, x, stream);
}

kq_status kq_draft_block_argmax_staged(const void *w_q4k, int layout, int64_t n, int64_t k, const void *staged,
                                       int verify_length, int32_t *proposals, int32_t *head_or_null,
                                       void *scratch, size_t scratch_bytes, void *stream) {
  if (!w_q4k || !staged || !proposals) return KQ_ERR_NULL;
  if (!verify_length_ok(verify_length)) return KQ_ERR_SHAPE;
  float *no_logits = nullptr;
  return run(&w_q4k, layout, 1, n, k, staged, verify_length + 1, &no_logits, true, nullptr, proposals, nullptr,
             1, head_or_null, scratch, scratch_bytes, nullptr, stream);
}

}  // extern "C"
