// Driver of the CPU sanitizer build of the host library (kq_api.cpp with the
// launcher stand-ins of kernel_stubs.cpp; built by g++ with
// -fsanitize=address,undefined and no recovery). It walks every entry point
// of include/kq.h through its argument checks (valid calls, which reach a
// stand-in launcher, and each refusal), the size functions over edge
// shapes, the chain encode / status path, and the host decision with the
// MT19937 stream on random inputs. Device pointers are placeholder addresses
// that the host code must never dereference: a dereference is a sanitizer
// error. Prints one line and exits 0 when every expectation holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "kq.h"
#include "stubs.h"

static int g_checks = 0, g_fail = 0;

#define EXPECT(cond)                                                         \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      ++g_fail;                                                              \
      fprintf(stderr, "host_check: line %d: %s\n", __LINE__, #cond);        \
    }                                                                        \
  } while (0)

// placeholder device addresses, 256-byte aligned, never dereferenced
static void *dev(uintptr_t i) { return reinterpret_cast<void *>((uintptr_t{1} << 44) + (i << 28)); }
template <class T>
static T *devp(uintptr_t i) { return static_cast<T *>(dev(i)); }

static void sizes() {
  const int64_t ns[] = {-1, 0, 1, 17, 6656, 131072, (int64_t)1 << 30, ((int64_t)1 << 31) - 1, (int64_t)1 << 31};
  const int64_t ks[] = {-256, 0, 255, 256, 6656, 33280, (int64_t)1 << 28, ((int64_t)1 << 28) + 256};
  const int ms[] = {-1, 0, 1, 15, 16, 17, 32, 33, 64, 65};
  for (int64_t n : ns)
    for (int64_t k : ks) {
      const size_t s = kq_scratch_bytes(n, k), t = kq_tiled_bytes(n, k);
      EXPECT((s == 0) == (t == 0));
      for (int layout = -1; layout <= 4; ++layout) (void)kq_tiled_bytes_fmt(layout, n, k);
      for (int c = -1; c <= 9; ++c) (void)kq_group_scratch_bytes(n, k, c);
      int waves = 0, tpw = 0, wg = 0;
      int64_t units = 0;
      const kq_status st = kq_launch_geometry(n, k, &waves, &tpw, &wg, &units);
      EXPECT(st == (s ? KQ_OK : KQ_ERR_SHAPE));
      if (st == KQ_OK) EXPECT(wg >= 1 && wg <= units && waves * tpw * 16 >= 128);
      for (int m : ms) (void)kq_workspace_bytes(n, k, m);
    }
  for (int64_t k : ks)
    for (int m : ms) (void)kq_staged_bytes_rows(k, m);
  for (int m : ms)
    for (int64_t n : ns) (void)kq_softmax_workspace_bytes(m, n);
  for (int p = -1; p <= 3; ++p) (void)kq_chain_table_bytes(p);
  EXPECT(kq_chain_table_bytes(KQ_MAX_CHAIN_PHASES + 1) == 0);
  for (int s = -1; s <= 7; ++s) EXPECT(kq_status_string(s) != nullptr);
}

static void products() {
  const int64_t n = 1000, k = 2304;
  const float *x = devp<const float>(1);
  float *logits = devp<float>(2);
  void *w = dev(3), *ws = dev(4), *staged = dev(5), *scratch = dev(6), *tiled = dev(7);
  int32_t *am = devp<int32_t>(8), *acc = devp<int32_t>(9), *path = devp<int32_t>(10);
  const size_t wsb = kq_workspace_bytes(n, k, 16), scb = kq_scratch_bytes(n, k);
  const size_t stb = kq_staged_bytes_rows(k, 64);
  int32_t draft[63];
  for (int i = 0; i < 63; ++i) draft[i] = (i * 37) % (int)n;

  const long g0 = kq::g_stub.gemv;
  EXPECT(kq_gemv_rows(w, n, k, x, 16, logits, ws, wsb, nullptr) == KQ_OK);
  EXPECT(kq_gemv_rows(w, n, k, x, 16, logits, ws, wsb - 1, nullptr) == KQ_ERR_WORKSPACE);
  EXPECT(kq_gemv_rows(nullptr, n, k, x, 16, logits, ws, wsb, nullptr) == KQ_ERR_NULL);
  EXPECT(kq_gemv_rows(w, n, k + 1, x, 16, logits, ws, wsb, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_gemv_rows((char *)w + 8, n, k, x, 16, logits, ws, wsb, nullptr) == KQ_ERR_ALIGN);
  for (int m = 1; m <= 16; ++m) {
    EXPECT(kq_verify_argmax_accept(w, n, k, x, m, draft, am, acc, nullptr, ws, kq_workspace_bytes(n, k, m),
                                   nullptr) == KQ_OK);
    EXPECT(kq_verify_argmax_accept_noalloc(w, n, k, x, m, draft, am, acc, logits, nullptr) == KQ_OK);
  }
  draft[3] = (int32_t)n;
  EXPECT(kq_verify_argmax_accept(w, n, k, x, 8, draft, am, acc, nullptr, ws, wsb, nullptr) == KQ_ERR_TOKEN);
  draft[3] = -1;
  EXPECT(kq_verify_argmax_accept_noalloc(w, n, k, x, 8, draft, am, acc, nullptr, nullptr) == KQ_ERR_TOKEN);
  draft[3] = 3;
  EXPECT(kq_verify_argmax_accept(w, n, k, x, 4, nullptr, am, acc, nullptr, ws, wsb, nullptr) == KQ_ERR_NULL);
  EXPECT(kq_verify_argmax_accept_noalloc(w, 1000, 512000, x, 16, draft, am, acc, nullptr, nullptr) ==
         KQ_ERR_WORKSPACE);

  EXPECT(kq_stage_rows(x, 64, k, staged, stb, nullptr) == KQ_OK);
  EXPECT(kq_stage_rows(x, 65, k, staged, stb, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_tile_weights(w, n, k, tiled, kq_tiled_bytes(n, k), nullptr) == KQ_OK);
  EXPECT(kq_tile_weights(w, n, k, w, kq_tiled_bytes(n, k), nullptr) == KQ_ERR_SHAPE);  // overlap
  for (int layout = KQ_LAYOUT_TILED16; layout <= KQ_LAYOUT_Q6K_TILED16; ++layout)
    EXPECT(kq_tile_weights_fmt(layout, w, n, k, tiled, kq_tiled_bytes_fmt(layout, n, k), nullptr) == KQ_OK);
  for (int layout = KQ_LAYOUT_ROWS; layout <= KQ_LAYOUT_Q6K_TILED16; ++layout)
    for (int m : {1, 7, 16, 17, 32, 48, 64}) {
      EXPECT(kq_gemv_staged(w, layout, n, k, staged, m, logits, scratch, scb, nullptr) == KQ_OK);
      if (m <= 16)
        EXPECT(kq_verify_staged(w, layout, n, k, staged, m, draft, am, acc, logits, scratch, scb, nullptr) ==
               KQ_OK);
      EXPECT(kq_verify_staged_dev(w, layout, n, k, staged, m, devp<int32_t>(11), am, acc, nullptr, scratch, scb,
                                  nullptr) == KQ_OK);
    }
  EXPECT(kq_gemv_staged(w, 4, n, k, staged, 4, logits, scratch, scb, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_gemv_staged(w, KQ_LAYOUT_ROWS, n, k, staged, 64, logits, scratch, scb - 256, nullptr) ==
         KQ_ERR_WORKSPACE);
  // a call of at most 16 rows needs only the one-slice part of the scratch
  const size_t sc1 = wsb - (kq_staged_bytes_rows(k, 16) + 255) / 256 * 256;
  EXPECT(sc1 < scb);
  EXPECT(kq_gemv_staged(w, KQ_LAYOUT_ROWS, n, k, staged, 4, logits, scratch, sc1, nullptr) == KQ_OK);
  EXPECT(kq_gemv_staged(w, KQ_LAYOUT_ROWS, n, k, staged, 4, logits, scratch, sc1 - 256, nullptr) ==
         KQ_ERR_WORKSPACE);
  for (int vl = 0; vl <= 16; ++vl) {
    const bool ok = vl == 3 || vl == 7 || vl == 15;
    EXPECT(kq_draft_block_argmax(w, n, k, x, vl, am, nullptr, ws, wsb, nullptr) == (ok ? KQ_OK : KQ_ERR_SHAPE));
    EXPECT(kq_draft_block_argmax_staged(w, KQ_LAYOUT_TILED16, n, k, staged, vl, am, acc, scratch, scb, nullptr) ==
           (ok ? KQ_OK : KQ_ERR_SHAPE));
  }
  // token trees: random parents before children, tokens in range; then each refusal
  std::mt19937 gen(7);
  for (int trial = 0; trial < 200; ++trial) {
    const int m = 1 + (int)(gen() % 64);
    std::vector<int32_t> parent(m), token(m);
    parent[0] = -1;
    token[0] = 12345;  // ignored
    for (int i = 1; i < m; ++i) {
      parent[i] = (int32_t)(gen() % i);
      token[i] = (int32_t)(gen() % n);
    }
    EXPECT(kq_verify_tree_staged(w, KQ_LAYOUT_TILED16, n, k, staged, m, parent.data(), token.data(), am, acc,
                                 trial % 2 ? path : nullptr, nullptr, scratch, scb, nullptr) == KQ_OK);
    if (m > 1) {
      const int j = 1 + (int)(gen() % (m - 1));
      const int32_t keep = parent[j];
      parent[j] = j;  // not before its child
      EXPECT(kq_verify_tree_staged(w, KQ_LAYOUT_TILED16, n, k, staged, m, parent.data(), token.data(), am, acc,
                                   nullptr, nullptr, scratch, scb, nullptr) == KQ_ERR_SHAPE);
      parent[j] = keep;
      token[j] = (int32_t)n;
      EXPECT(kq_verify_tree_staged(w, KQ_LAYOUT_TILED16, n, k, staged, m, parent.data(), token.data(), am, acc,
                                   nullptr, nullptr, scratch, scb, nullptr) == KQ_ERR_TOKEN);
    }
  }
  // grouped launches of 1 .. 8 matrices, then 0 and 9
  const void *ws8[KQ_MAX_GROUP + 1];
  float *lg8[KQ_MAX_GROUP + 1];
  for (int i = 0; i <= KQ_MAX_GROUP; ++i) {
    ws8[i] = dev(20 + i);
    lg8[i] = devp<float>(40 + i);
  }
  for (int c = 0; c <= KQ_MAX_GROUP + 1; ++c) {
    const size_t gb = kq_group_scratch_bytes(n, k, c);
    const kq_status st = kq_gemv_staged_group(ws8, KQ_LAYOUT_TILED16, c, n, k, staged, 16, lg8, scratch,
                                              gb ? gb : scb, nullptr);
    EXPECT(st == (c >= 1 && c <= KQ_MAX_GROUP ? KQ_OK : KQ_ERR_SHAPE));
  }
  EXPECT(kq::g_stub.gemv > g0 + 300);

  // softmax rows, gather, stream probe, workspace init
  const size_t smb = kq_softmax_workspace_bytes(16, 131072);
  EXPECT(kq_softmax_rows(x, 16, 131072, 0.7f, 30.0f, logits, ws, smb, nullptr) == KQ_OK);
  EXPECT(kq_softmax_rows(x, 16, 131072, 0.0f, 30.0f, logits, ws, smb, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_softmax_rows(x, 16, 131072, 0.7f, -1.0f, logits, ws, smb, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_softmax_rows(x, 16, 131072, 0.7f, 0.0f, logits, ws, smb - 256, nullptr) == KQ_ERR_WORKSPACE);
  EXPECT(kq_gather_rows(x, 16, 131072, am, 16, logits, nullptr) == KQ_OK);
  EXPECT(kq_gather_rows(x, 16, 131072, am, 17, logits, nullptr) == KQ_ERR_SHAPE);
  EXPECT(kq_gather_rows(nullptr, 16, 131072, am, 0, logits, nullptr) == KQ_OK);
  EXPECT(kq_stream_probe(w, 1 << 20, devp<uint32_t>(12), kq_stream_probe_sink_bytes(), nullptr) == KQ_OK);
  EXPECT(kq_stream_probe(w, (1 << 20) + 8, devp<uint32_t>(12), kq_stream_probe_sink_bytes(), nullptr) ==
         KQ_ERR_SHAPE);
  EXPECT(kq_workspace_init(ws, wsb, nullptr) == KQ_OK);
  EXPECT(kq_workspace_init(nullptr, wsb, nullptr) == KQ_ERR_NULL);
}

static void chains() {
  const int64_t shapes[4][3] = {{3, 6656, 6656}, {1, 6656, 6656}, {2, 17920, 6656}, {1, 6656, 17920}};
  std::vector<kq_chain_phase> ph(8);
  for (int i = 0; i < 8; ++i) {
    memset(&ph[i], 0, sizeof ph[i]);
    ph[i].count = (int)shapes[i % 4][0];
    ph[i].n = shapes[i % 4][1];
    ph[i].k = shapes[i % 4][2];
    for (int j = 0; j < ph[i].count; ++j) {
      ph[i].w_q4k[j] = dev(60 + 8 * i + j);
      ph[i].logits[j] = devp<float>(200 + 8 * i + j);
    }
    ph[i].staged = dev(400 + (ph[i].k == 6656 ? 0 : 1));
  }
  const size_t tb = kq_chain_table_bytes(8);
  std::vector<unsigned char> table(tb + 64);
  for (int m : {1, 16}) {
    kq_chain_plan plan;
    memset(&plan, 0, sizeof plan);
    EXPECT(kq_chain_encode(ph.data(), 8, m, KQ_LAYOUT_TILED16, table.data(), tb, &plan) == KQ_OK);
    EXPECT(plan.n_phases == 8 && plan.m == m && plan.workgroups >= 1 && plan.workgroups <= 256);
    EXPECT(plan.table_bytes == tb && plan.scratch_bytes > 0);
    void *sc = dev(500);
    EXPECT(kq_chain_scratch_init(&plan, sc, plan.scratch_bytes, nullptr) == KQ_OK);
    EXPECT(kq_gemv_chain(dev(501), &plan, sc, plan.scratch_bytes, nullptr) == KQ_OK);
    EXPECT(kq_gemv_chain(dev(501), &plan, sc, plan.scratch_bytes - 1, nullptr) == KQ_ERR_WORKSPACE);
    kq::g_stub.device_word = 0;
    EXPECT(kq_chain_status(&plan, sc, plan.scratch_bytes, nullptr) == KQ_OK);
    kq::g_stub.device_word = 1;
    EXPECT(kq_chain_status(&plan, sc, plan.scratch_bytes, nullptr) == KQ_ERR_LAUNCH);
    kq::g_stub.device_word = 0;
    kq_chain_plan bad = plan;
    bad.tiles_per_wave = 2;
    EXPECT(kq_gemv_chain(dev(501), &bad, sc, plan.scratch_bytes, nullptr) == KQ_ERR_SHAPE);
    EXPECT(kq_chain_status(&bad, sc, plan.scratch_bytes, nullptr) == KQ_ERR_SHAPE);
  }
  kq_chain_plan plan;
  EXPECT(kq_chain_encode(ph.data(), 8, 16, KQ_LAYOUT_Q5K_TILED16, table.data(), tb, &plan) == KQ_ERR_SHAPE);
  EXPECT(kq_chain_encode(ph.data(), 8, 16, KQ_LAYOUT_TILED16, table.data(), tb - 1, &plan) == KQ_ERR_WORKSPACE);
  ph[5].w_q4k[0] = nullptr;
  EXPECT(kq_chain_encode(ph.data(), 8, 16, KQ_LAYOUT_TILED16, table.data(), tb, &plan) == KQ_ERR_NULL);
  ph[5].w_q4k[0] = dev(99);
  ph[2].k = 6657;
  EXPECT(kq_chain_encode(ph.data(), 8, 16, KQ_LAYOUT_TILED16, table.data(), tb, &plan) == KQ_ERR_SHAPE);
}

static void decisions() {
  kq_mt19937 g;
  EXPECT(kq_mt19937_seed(&g, 5489u) == KQ_OK);
  std::vector<uint32_t> words(10000);
  EXPECT(kq_mt19937_u32(&g, words.data(), 10000) == KQ_OK);
  EXPECT(words[9999] == 4123659995u);
  std::mt19937 gen(123);
  for (int trial = 0; trial < 400; ++trial) {
    const int k = (int)(gen() % 16), n = 1 + (int)(gen() % 300);
    std::vector<float> q((size_t)(k ? k : 1) * n), p((size_t)(k + 1) * n), u(k + 1);
    std::vector<int32_t> orders((size_t)(k + 1) * n), draft(k + 1);
    std::uniform_real_distribution<float> uni(0.0f, 1.0f);
    for (auto &v : q) v = uni(gen) < 0.2f ? 0.0f : uni(gen);
    for (auto &v : p) v = uni(gen) < 0.2f ? 0.0f : uni(gen);
    if (trial % 3 == 0)
      for (int i = 0; i < k * n; ++i) q[i] = p[i];  // certain acceptance
    for (int r = 0; r <= k; ++r) {
      for (int j = 0; j < n; ++j) orders[(size_t)r * n + j] = j;
      std::shuffle(orders.begin() + (size_t)r * n, orders.begin() + (size_t)(r + 1) * n, gen);
    }
    for (int i = 0; i < k; ++i) draft[i] = (int32_t)(gen() % n);
    kq_mt19937 s, ahead;
    kq_mt19937_seed(&s, (uint32_t)gen());
    ahead = s;
    EXPECT(kq_mt19937_uniform_f32(&ahead, u.data(), k + 1) == KQ_OK);
    int32_t a1 = -1, t1 = -1, a2 = -2, t2 = -2;
    const kq_status s1 =
        kq_speculative_decide(k, draft.data(), n, q.data(), p.data(), orders.data(), u.data(), &a1, &t1);
    const kq_status s2 = kq_speculative_decide_mt(k, draft.data(), n, q.data(), p.data(), orders.data(), &s, &a2, &t2);
    EXPECT(s1 == s2);
    if (s1 == KQ_OK) {
      EXPECT(a1 == a2 && t1 == t2 && a1 >= 0 && a1 <= k && t1 >= 0 && t1 < n);
      int32_t pos = -1;
      std::vector<float> pa(k + 1), qa(k + 1);
      for (int i = 0; i < k; ++i) {
        pa[i] = p[(size_t)i * n + draft[i]];
        qa[i] = q[(size_t)i * n + draft[i]];
      }
      EXPECT(kq_speculative_first_reject(k, pa.data(), qa.data(), u.data(), &pos) == KQ_OK && pos == a1);
    }
    int32_t tok = -1;
    (void)kq_speculative_resample(n, p.data(), trial % 2 ? q.data() : nullptr, orders.data(), u[0], &tok);
  }
  int32_t a = 0, t = 0;
  EXPECT(kq_speculative_decide_mt(3, nullptr, 10, nullptr, nullptr, nullptr, &g, &a, &t) == KQ_ERR_NULL);
  EXPECT(kq_speculative_decide_mt(3, nullptr, 10, nullptr, nullptr, nullptr, nullptr, &a, &t) == KQ_ERR_NULL);
  EXPECT(kq_mt19937_u32(&g, nullptr, -1) == KQ_ERR_SHAPE);
}

int main() {
  memset(&kq::g_stub, 0, sizeof kq::g_stub);
  sizes();
  products();
  chains();
  decisions();
  if (kq::g_stub.violation[0]) {
    fprintf(stderr, "host_check: launch invariant: %s\n", kq::g_stub.violation);
    ++g_fail;
  }
  printf("host_check: %d checks, %d failed; launches: gemv %ld stage %ld fill %ld tile %ld softmax %ld\n", g_checks,
         g_fail, kq::g_stub.gemv, kq::g_stub.stage, kq::g_stub.fill, kq::g_stub.tile, kq::g_stub.softmax);
  return g_fail ? 1 : 0;
}
