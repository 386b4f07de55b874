// Host-only stand-ins for the kernel launchers of kq_kernels.hip, for the
// CPU sanitizer build of kq_api.cpp (AddressSanitizer + UndefinedBehavior-
// Sanitizer with g++; no HIP runtime, no device). Each launcher enqueues
// nothing: it counts the call and checks the launch description it was
// given against the invariants the kernels rely on, recording the first
// violation for the driver to report. Device pointers are never
// dereferenced (the driver passes placeholder addresses).
#include <stdio.h>
#include <string.h>

#include "kq_internal.h"
#include "stubs.h"

namespace kq {

StubLog g_stub;

static void violate(const char *what) {
  if (!g_stub.violation[0]) snprintf(g_stub.violation, sizeof g_stub.violation, "%s", what);
}

int launch_stage(const float *x, int m, int64_t k, uint8_t *staged, unsigned *ctrl, int64_t n_groups, void *) {
  ++g_stub.stage;
  if (!x || !staged || m < 1 || m > kMaxTreeRows || k < kQK || k % kQK) violate("stage: bad arguments");
  if (ctrl && n_groups < 1) violate("stage: control words without row groups");
  return 0;
}

int launch_gemv(const GemvLaunch &a, void *) {
  ++g_stub.gemv;
  const Geometry &g = a.g;
  if (a.m < 1 || a.m > kMaxTreeRows) violate("gemv: m out of range");
  if (a.chain) {
    if (a.n_phases < 1 || !a.bar || !a.err || !a.epoch || !a.flags || !a.partials) violate("gemv: chain words");
    return 0;
  }
  if (g.count < 1 || g.count > kMaxGroup || g.kb < 1 || g.rows != 16 * g.waves * g.tpw) violate("gemv: geometry");
  if (g.units != (int64_t)g.n_groups * g.kb || g.n_wg < 1 || g.n_wg > g.units) violate("gemv: unit split");
  if (g.n_groups != g.count * g.n_wg_per || (int64_t)g.n_wg_per * g.rows < a.ph.n) violate("gemv: row groups");
  for (int i = 0; i < g.count; ++i)
    if (!a.ph.w[i]) violate("gemv: null weight pointer");
  if (!a.ph.staged || !a.partials || !a.done || !a.group_cnt || !a.wg_keys) violate("gemv: null scratch part");
  if (a.verify && (!a.argmax_out || a.k_draft < 0 || a.k_draft >= kMaxTreeRows)) violate("gemv: verify outputs");
  return 0;
}

int chain_capacity() { return 256; }

int launch_fill(unsigned *p, int64_t n_words, void *, unsigned) {
  ++g_stub.fill;
  if (!p || n_words < 0) violate("fill: bad arguments");
  return 0;
}

int read_device_word(const unsigned *dev, unsigned *host, void *) {
  ++g_stub.read;
  if (!dev || !host) violate("read: bad arguments");
  *host = g_stub.device_word;
  return 0;
}

int noalloc_workspace(void **ptr) {
  *ptr = reinterpret_cast<void *>(static_cast<uintptr_t>(1) << 40);
  return 0;
}

int launch_tile(const uint8_t *w, int64_t n, int64_t k, uint8_t *out, void *, int fmt) {
  ++g_stub.tile;
  if (!w || !out || n < 1 || k < kQK || fmt < kFmtQ4 || fmt > kFmtQ6) violate("tile: bad arguments");
  return 0;
}

int launch_stream_probe(const uint8_t *p, int64_t chunks, unsigned *sink, int blocks, void *) {
  ++g_stub.probe;
  if (!p || !sink || chunks < 1 || blocks < 1) violate("probe: bad arguments");
  return 0;
}

int softmax_chunks(int64_t n) { return (int)((n + 4095) / 4096); }

int launch_gather(const float *rows, int64_t n, const int32_t *tokens, int count, float *out, void *) {
  ++g_stub.gather;
  if (!rows || !tokens || !out || n < 1 || count < 1) violate("gather: bad arguments");
  return 0;
}

int launch_softmax(const float *logits, int m, int64_t n, float temperature, float, float *part, float *probs,
                   void *) {
  ++g_stub.softmax;
  if (!logits || !part || !probs || m < 1 || n < 1 || !(temperature > 0)) violate("softmax: bad arguments");
  return 0;
}

}  // namespace kq
