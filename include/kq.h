/*
 * kq.h -- C ABI of libkq: the k-quant (Q4_K, Q5_K, Q6_K) batched
 * speculative-verify step on MI355X (gfx950): the skinny products, the fused
 * argmax and greedy accept (linear or over a token tree), the draft block's
 * proposals, chains of dependent products in one launch, and the stochastic
 * verify's probability rows and host decision.
 *
 * The operation (muser-book ch. 33 "Speculation: the local win and the
 * distributed verdict", section 33.1; ch. 8 "The DFlash draft", section 8.1):
 * a draft proposes k tokens and the target scores all k+1 positions in one
 * pass over its weights, k+1 activation rows per weight read. For a Q4_K
 * weight matrix W with N output rows of K weights and M = k+1 fp32 rows x,
 *
 *     logits[m][n] = sum_k W[n][k] * x[m][k]
 *
 * where W is decoded on the fly from 144-byte, 256-weight super-blocks
 * (w = d * sc_j * q - dmin * m_j; fp16 d/dmin, 6-bit sub-block scales and
 * mins, 4-bit quants; the llama.cpp GGUF layout). The pages name the format
 * and say kquant matrices are consumed in place, never expanded (ch. 8,
 * sections 8.2 and 8.5); this library reads the raw block bytes.
 *
 * The verify call also takes each row's argmax ("the index of each row's
 * largest score", ch. 8 section 8.6; ties -> lowest index) and applies the
 * greedy accept rule, the temperature-0 limit of the accept/resample rule of
 * ch. 33 section 33.2: accepted = first i < k with draft[i] != argmax[i]
 * (k if none), next_token = argmax[accepted], emitted = accepted + 1.
 *
 * Conventions (all entry points):
 *  - Shapes: 1 <= m <= 64 (more than 16 only where stated: not for chains
 *    or the draft block), k > 0 and k % 256 == 0, k <= 2^28, 1 <= n < 2^31,
 *    and the weight matrix (n rounded up to a multiple of 16) and the staged
 *    activations each smaller than 4 GiB: ceil(n/16) * 16 * (k/256) * (block
 *    bytes) < 2^32 and kq_staged_bytes_rows(k, m) < 2^32 (the kernels
 *    address them with 32-bit offsets). Other shapes give KQ_ERR_SHAPE (size
 *    queries return 0).
 *  - Layouts: w is [n][k/256] Q4_K blocks of 144 bytes, row-major, 16-byte
 *    aligned, or one of the tiled layouts below; x is fp32 [m][k]
 *    row-major, 16-byte aligned; logits fp32 [m][n].
 *  - Pointers marked "device" are HIP device memory owned by the caller; the
 *    library allocates nothing and keeps no global mutable state, except the
 *    fixed workspace of kq_verify_argmax_accept_noalloc (a device array per
 *    GPU and its looked-up address, see there).
 *  - Every call is enqueued on `stream` (a hipStream_t; NULL = default
 *    stream) and returns without synchronising; results are valid once the
 *    stream reaches that point.
 *  - Errors: every argument check runs before any HIP call; on a non-OK
 *    return nothing has been enqueued. KQ_ERR_LAUNCH reports a HIP launch
 *    failure (hipGetLastError after enqueue).
 *  - Concurrency: calls on different streams need different workspaces;
 *    calls sharing a workspace must be ordered (e.g. the same stream).
 *  - Numerics: every product of a weight operand and an activation operand
 *    is exact (fp16 x fp16, the activations split into an exact fp16 pair),
 *    sums are fp32. The scale term d sc_j q_k and the min term dmin m_j of
 *    each weight are contracted apart and subtracted once per 256-column
 *    block, so the rounding error is bounded by the mass of both terms,
 *    B = sum_k (|d sc_j q_k| + |dmin m_j|) |x_k| (B = sum_k |w_k x_k| for
 *    Q6_K, which has no min term):
 *        |logit - exact| <= 2^-24 (544 + k/128) B
 *    for finite inputs with |dmin| * 63 <= 65504 (a worst case that lets
 *    every fp32 addition round; activations smaller than 2^-12 of the
 *    largest magnitude of their row in their 256-column block may each add
 *    an absolute error of 2^-34 of that magnitude times their weight's term
 *    mass). This guarantees the tolerance 1e-4 * sum_k |w_k x_k| whenever B
 *    is at most 2 times sum_k |w_k x_k| (k <= 33,280), which covers weights
 *    that are mostly of one sign (every configured workload: B is about 1.3
 *    times that mass). Weights centred on zero, as quantizers fit real
 *    weights (B about 4 times), are outside that guarantee but are held to
 *    the tolerance by the tests (tests/test_gpu_cancel.py). Weights whose
 *    two terms cancel (w = 0 with d, dmin nonzero) contribute to B but not
 *    to the tolerance, so a row of them can exceed 1e-4 * sum_k |w_k x_k|,
 *    never the bound above. Results are bitwise deterministic, and for
 *    m <= 16 row i of an m-row call equals the 1-row call on x[i] bit for
 *    bit (calls of more than 16 rows may cut the work differently; they
 *    meet the same bound). A call of 33 to 64 rows equals a 32-row call on
 *    rows 0-31 and a call on the remaining rows, bit for bit. There is no
 *    CPU or alternate path.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int kq_status;
#define KQ_OK            0
#define KQ_ERR_NULL      1  /* a required pointer is NULL                       */
#define KQ_ERR_SHAPE     2  /* m, n or k out of range                           */
#define KQ_ERR_ALIGN     3  /* w, x, staged or workspace not 16/256-byte aligned */
#define KQ_ERR_TOKEN     4  /* a draft token outside [0, n)                     */
#define KQ_ERR_WORKSPACE 5  /* workspace / staged buffer smaller than required  */
#define KQ_ERR_LAUNCH    6  /* HIP reported an error when enqueuing             */

/* Weight layouts accepted by the staged calls. */
#define KQ_LAYOUT_ROWS    0  /* llama.cpp: row n is k/256 consecutive 144-byte blocks */
#define KQ_LAYOUT_TILED16 1  /* kq_tile_weights output (same bytes, reordered) */
/* Q5_K and Q6_K weights (the draft loads Q4_K, Q5_K and Q6_K tensors and its
 * v projection is Q6_K: muser-book ch. 8 "The DFlash draft", section 8.2),
 * tiled by kq_tile_weights_fmt from llama.cpp rows (176- and 210-byte
 * blocks); every entry point that takes a layout accepts them. */
#define KQ_LAYOUT_Q5K_TILED16 2
#define KQ_LAYOUT_Q6K_TILED16 3

/* Measurement helper, not part of the verify step: reads every byte of a
 * device buffer once (16-byte loads over the whole GPU) and writes one
 * XOR-fold word per workgroup to `sink`, so a caller can time the HBM read
 * rate the weight stream could reach on this device (a benchmark reports it
 * next to the roofline).
 *  buf   device, `bytes` bytes, 16-byte aligned, bytes % 16 == 0 (else KQ_ERR_SHAPE)
 *  sink  device, >= kq_stream_probe_sink_bytes() bytes (written; contents
 *        are a checksum, not a result) */
size_t kq_stream_probe_sink_bytes(void);
kq_status kq_stream_probe(const void *buf, size_t bytes, uint32_t *sink, size_t sink_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *kq_status_string(kq_status s);

/* Bytes of device workspace kq_gemv_rows / kq_verify_argmax_accept need for
 * an n x k matrix and m rows (0 for invalid shapes). The workspace holds the
 * staged activations, split-K partial sums and the control words; it grows
 * with the number of 16-row slices of m (at m = 64 it is the staged bytes,
 * rounded up to 256, plus kq_scratch_bytes(n, k)). */
size_t kq_workspace_bytes(int64_t n, int64_t k, int m);

/* Bytes of a staged activation block for k columns (any m <= 16). */
size_t kq_staged_bytes(int64_t k);

/* Bytes of a staged activation block for m <= 64 rows of k columns (0 for
 * invalid arguments): (k/256) * s * 16,960 with s = ceil(m/16) sixteen-row
 * slices (1 to 4). Calls of 17 to 64 rows (the token-tree verify,
 * kq_verify_tree_staged, or a longer linear verify) run every weight tile
 * against all s slices in the same pass, in every format, so the weights
 * are still read once per call. */
size_t kq_staged_bytes_rows(int64_t k, int m);

/* Bytes of device scratch the *_staged calls need for an n x k matrix (in
 * any weight format and layout). The scratch is laid out for the shape
 * alone: every single-matrix call on n x k may share it (any format,
 * layout and m, ordered on one stream). A call on another shape, or a
 * grouped call, needs its own scratch, or this one zeroed again with
 * kq_workspace_init first. The size covers calls of up to 64 rows; a call
 * refuses (KQ_ERR_WORKSPACE) only a scratch smaller than its own m needs
 * (its split-K partial sums grow with the 16-row slices of m). */
size_t kq_scratch_bytes(int64_t n, int64_t k);

/* Zero the control words of a workspace or scratch buffer of `bytes` bytes
 * (device, 256-byte aligned). Scratch passed to the *_staged calls must be
 * zeroed once before first use; every call leaves it zeroed again.
 * kq_gemv_rows / kq_verify_argmax_accept re-zero their workspace themselves. */
kq_status kq_workspace_init(void *workspace, size_t bytes, void *stream);

/* Logits of m activation rows against one Q4_K matrix.
 *  w_q4k      device, n * (k/256) * 144 bytes (read only)
 *  x          device, fp32 [m][k] (read only)
 *  logits     device, fp32 [m][n] (written)
 *  workspace  device, >= kq_workspace_bytes(n, k, m) bytes, 256-byte aligned
 * Passage: ch. 33 section 33.1 / ch. 8 section 8.1 (k+1 rows per weight read);
 * the same call serves the draft's fc projection 33,280 -> 6,656 of five
 * concatenated target hidden states (ch. 8 section 8.2). */
kq_status kq_gemv_rows(const void *w_q4k, int64_t n, int64_t k,
                       const float *x, int m, float *logits,
                       void *workspace, size_t workspace_bytes, void *stream);

/* The verify step: logits (optional), per-row argmax and greedy accept.
 *  m               k_draft + 1 (1..64): row i < m-1 judges draft[i], row
 *                  m-1 supplies the token after a full accept
 *  draft_host      host, m-1 int32 tokens in [0, n) (copied before return;
 *                  may be NULL when m == 1)
 *  argmax          device, int32 [m] (written)
 *  accept_out      device, int32 [2] = {accepted, next_token} (written)
 *  logits_or_null  device fp32 [m][n], or NULL to skip writing logits
 * Passages: ch. 33 section 33.2 (accept rule, greedy limit), ch. 8 section
 * 8.6 (argmax of each row). */
kq_status kq_verify_argmax_accept(const void *w_q4k, int64_t n, int64_t k,
                                  const float *x, int m,
                                  const int32_t *draft_host,
                                  int32_t *argmax, int32_t *accept_out,
                                  float *logits_or_null,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* kq_verify_argmax_accept without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). The workspace is a
 * file-scope device array of KQ_NOALLOC_MAX_BYTES inside the library, one
 * per GPU (held until the process ends); its address is looked up once per
 * device, on the first call with that device current. Nothing is allocated.
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (different streams, or different threads without ordering) race and
 * give wrong results; calls ordered on one stream are safe. Each call
 * re-zeroes the control words it needs, so the array's earlier contents
 * do not matter. Arguments as for kq_verify_argmax_accept; KQ_ERR_WORKSPACE
 * (before any HIP call) when kq_workspace_bytes(n, k, m) exceeds
 * KQ_NOALLOC_MAX_BYTES; KQ_ERR_LAUNCH when the address lookup fails. */
#define KQ_NOALLOC_MAX_BYTES (24u << 20)
kq_status kq_verify_argmax_accept_noalloc(const void *w_q4k, int64_t n, int64_t k,
                                          const float *x, int m,
                                          const int32_t *draft_host,
                                          int32_t *argmax, int32_t *accept_out,
                                          float *logits_or_null, void *stream);

/* Stage m fp32 activation rows once for any number of matrices with the same
 * k (projections that share an input: q/k/v, gate/up).
 *  x       device, fp32 [m][k]
 *  m       1..64 (more than 16: see kq_staged_bytes_rows)
 *  staged  device, >= kq_staged_bytes_rows(k, m) bytes (kq_staged_bytes(k)
 *          for m <= 16), 256-byte aligned (written)
 * A staged block is valid for the m it was staged with. */
kq_status kq_stage_rows(const float *x, int m, int64_t k,
                        void *staged, size_t staged_bytes, void *stream);

/* Bytes of the tiled copy of an n x k Q4_K matrix (0 for invalid shapes):
 * ceil(n/16) * (k/256) * 2,304. */
size_t kq_tiled_bytes(int64_t n, int64_t k);

/* Reorder the bytes of an n x k Q4_K matrix (llama.cpp layout, device) into
 * KQ_LAYOUT_TILED16 (device, >= kq_tiled_bytes(n, k) bytes, 16-byte aligned,
 * not overlapping the input). Every byte of every 144-byte block is kept;
 * only their order changes: record (b, t) = block b of the 16-row tile t
 * (rows 16t .. 16t+15) is 2,304 bytes at (b * ceil(n/16) + t) * 2,304 and
 * holds the 16 block headers (row order), then quant bytes [16g, 16g+16) of
 * row r at 256 + 16 (16 g + r) and quant bytes [64+16g, 80+16g) of row r at
 * 1,280 + 16 (16 g + r), g = 0..3. Rows past n are zero. All blocks of one
 * 256-column block index for consecutive rows are contiguous, so each wave
 * reads whole cache lines. One-time preparation of resident weights; the
 * staged calls accept either layout and give bitwise identical results.
 * Overlapping input and output buffers are refused with KQ_ERR_SHAPE. */
kq_status kq_tile_weights(const void *w_q4k, int64_t n, int64_t k,
                          void *w_tiled, size_t tiled_bytes, void *stream);

/* Bytes of the tiled copy in `layout` (KQ_LAYOUT_TILED16, KQ_LAYOUT_Q5K_TILED16
 * or KQ_LAYOUT_Q6K_TILED16) of an n x k matrix: ceil(n/16) * (k/256) * 16 *
 * (144, 176 or 210); 0 for invalid shapes or layouts. */
size_t kq_tiled_bytes_fmt(int layout, int64_t n, int64_t k);

/* Tile an n x k matrix given as llama.cpp rows of its format (device; Q4_K
 * 144-, Q5_K 176-, Q6_K 210-byte blocks, layout GGUF) into `layout`
 * (device, >= kq_tiled_bytes_fmt bytes, 16-byte aligned, not overlapping the
 * input). KQ_LAYOUT_TILED16 is kq_tile_weights. The Q5_K and Q6_K records
 * (block b of 16-row tile t at (b * ceil(n/16) + t) * 16 * block bytes) keep
 * every bit of the 16 blocks, reordered so that lane l = 16 g + r of a wave
 * (row r, g = 0..3) reads its weights' low four bits exactly where a Q4_K
 * record keeps them:
 *  Q5_K (2,816 B): the 16 headers (d, dmin, 12 scale/min bytes) at 16 r;
 *    quant bytes [16g, 16g+16) at 256 + 16 l and [64+16g, 80+16g) at
 *    1,280 + 16 l; the lane's 64 fifth bits at 2,304 + 8 l.
 *  Q6_K (3,360 B): the lane's 4 signed scales at 4 l; the low nibbles in the
 *    Q4_K order at 256 + 16 l and 1,280 + 16 l; the lane's 64 two-bit high
 *    parts at 2,304 + 16 l; fp16 d of row r at 3,328 + 2 r.
 * Rows past n are zero. Q5_K and Q6_K have no row-major kernel path: pass
 * their tiled copy. Input the row layout requires: the rows are 16-byte
 * aligned for Q4_K and Q5_K, 2-byte aligned for Q6_K. */
kq_status kq_tile_weights_fmt(int layout, const void *w_rows, int64_t n, int64_t k,
                              void *w_tiled, size_t tiled_bytes, void *stream);

/* kq_gemv_rows on staged activations (every staged call: `staged` comes from
 * kq_stage_rows with the same m, since its size and slice layout depend on
 * m).
 *  layout   KQ_LAYOUT_ROWS or KQ_LAYOUT_TILED16 (the layout of w_q4k), or
 *           KQ_LAYOUT_Q5K_TILED16 / KQ_LAYOUT_Q6K_TILED16 (w_q4k is then a
 *           tiled Q5_K or Q6_K matrix; same staged activations)
 *  scratch  device, >= kq_scratch_bytes(n, k) bytes, 256-byte aligned,
 *           zeroed once by kq_workspace_init */
kq_status kq_gemv_staged(const void *w_q4k, int layout, int64_t n, int64_t k,
                         const void *staged, int m, float *logits,
                         void *scratch, size_t scratch_bytes, void *stream);

/* Draft block proposals (ch. 8 section 8.6, guarantee 3; the 16-row block of
 * section 8.2). The draft forwards one 16-row block (a seed row followed by 15
 * mask rows), scores the block's output rows with the target's LM head and
 * proposes the argmax (ties -> lowest index) of rows 1..verify_length; the
 * verify length is exactly 3, 7 or 15, and any other value is an error
 * before any GPU work. Only rows 0..verify_length are scored (the weight
 * stream, and so the cost, does not depend on how many).
 *  w_q4k          device, the LM head, n * (k/256) * 144 bytes (read only)
 *  x              device, fp32 [>= verify_length + 1][k]: the block's output
 *                 rows; rows past verify_length are not read
 *  verify_length  3, 7 or 15 (else KQ_ERR_SHAPE)
 *  proposals      device, int32 [verify_length] (written): argmax of rows
 *                 1..verify_length, in row order
 *  head_or_null   device int32 [1] (written: argmax of row 0, the block head
 *                 the pages check against the seed token) or NULL
 *  workspace      >= kq_workspace_bytes(n, k, verify_length + 1) bytes, as for
 *                 kq_verify_argmax_accept
 * Argmax rows whose top-2 gap lies inside the logit tolerance may resolve to
 * any of the tied candidates (as in the verify step). */
kq_status kq_draft_block_argmax(const void *w_q4k, int64_t n, int64_t k,
                                const float *x, int verify_length,
                                int32_t *proposals, int32_t *head_or_null,
                                void *workspace, size_t workspace_bytes, void *stream);

/* kq_draft_block_argmax on staged activations (staged holds at least rows
 * 0..verify_length of the block, kq_stage_rows); layout and scratch as for
 * kq_gemv_staged. */
kq_status kq_draft_block_argmax_staged(const void *w_q4k, int layout, int64_t n, int64_t k,
                                       const void *staged, int verify_length,
                                       int32_t *proposals, int32_t *head_or_null,
                                       void *scratch, size_t scratch_bytes, void *stream);

/* kq_verify_argmax_accept on staged activations (same arguments as above;
 * layout and scratch as for kq_gemv_staged). */
kq_status kq_verify_staged(const void *w_q4k, int layout, int64_t n, int64_t k,
                           const void *staged, int m,
                           const int32_t *draft_host,
                           int32_t *argmax, int32_t *accept_out,
                           float *logits_or_null,
                           void *scratch, size_t scratch_bytes, void *stream);

/* kq_verify_staged with the draft tokens in device memory (for drafts the
 * GPU produced, e.g. kq_draft_block_argmax_staged's proposals: draft and
 * verify then run on one stream with no host round trip).
 *  draft_dev  device int32 [m-1], 4-byte aligned (may be NULL when m == 1);
 *             read by the kernel, so the tokens are not range-checked on
 *             the host: a token outside [0, n) never equals a row's argmax,
 *             and so counts as a mismatch (it is only compared, never used
 *             as an index). */
kq_status kq_verify_staged_dev(const void *w, int layout, int64_t n, int64_t k, const void *staged, int m,
                               const int32_t *draft_dev, int32_t *argmax, int32_t *accept_out,
                               float *logits_or_null, void *scratch, size_t scratch_bytes, void *stream);

/* Token-tree verify (ch. 33 "Speculation: the local win and the
 * distributed verdict", section 33.7: the hardware-aware token tree spends
 * the batch arithmetic a weight stream leaves idle on near-miss branches,
 * at 24, 32, 48 or 64 nodes). One pass over the weights scores all m nodes
 * (m <= 64; activation row i is node i's position),
 * takes every row's argmax (ties -> lowest index) and walks the tree: from
 * the root (node 0), move to a child whose token equals the current node's
 * argmax (the lowest index when siblings repeat a token) until none does.
 *  staged        kq_stage_rows of the m node rows (kq_staged_bytes_rows)
 *  parent_host   host int32 [m]: parent_host[0] = -1, parent_host[i] in
 *                [0, i) (parents before children), else KQ_ERR_SHAPE
 *  token_host    host int32 [m]: the token node i proposes (i >= 1, in
 *                [0, n), else KQ_ERR_TOKEN); entry 0 is ignored
 *  argmax        device int32 [m] (written)
 *  accept_out    device int32 [2] = {nodes moved through, the argmax of the
 *                node where the walk stops} (written)
 *  path_out_or_null  device int32 [m] or NULL: entries 0..accepted-1 are the
 *                nodes moved through, in order (the rest untouched)
 *  logits_or_null, scratch: as kq_verify_staged. A chain (parent i - 1)
 * gives kq_verify_staged's result for the same tokens. Every argument is
 * checked before any HIP call. */
kq_status kq_verify_tree_staged(const void *w, int layout, int64_t n, int64_t k, const void *staged, int m,
                                const int32_t *parent_host, const int32_t *token_host, int32_t *argmax,
                                int32_t *accept_out, int32_t *path_out_or_null, float *logits_or_null,
                                void *scratch, size_t scratch_bytes, void *stream);

/* Bytes of device scratch kq_gemv_staged_group needs for `count` matrices
 * of n x k in any weight format (0 for invalid arguments).
 * The layout depends on n, k and count: calls with another shape or count
 * need their own scratch, or this one zeroed again with kq_workspace_init. */
size_t kq_group_scratch_bytes(int64_t n, int64_t k, int count);

/* kq_gemv_staged for 1 <= count <= 8 matrices of the same shape that share
 * the staged activations (projections of one input, e.g. q/k/v or gate/up),
 * in one launch.
 *  w_q4k   host array of `count` device pointers (each 16-byte aligned), all
 *          in `layout` (KQ_LAYOUT_ROWS or KQ_LAYOUT_TILED16)
 *  logits  host array of `count` device pointers, fp32 [m][n] each
 *  scratch device, >= kq_group_scratch_bytes(n, k, count) bytes, zeroed once
 * Each matrix's logits are deterministic and within the kq.h tolerance; they
 * may differ in the last bits from a separate kq_gemv_staged call because the
 * launch can divide k differently among workgroups (the division depends on
 * n, k and count). */
kq_status kq_gemv_staged_group(const void *const *w_q4k, int layout, int count, int64_t n, int64_t k,
                               const void *staged, int m, float *const *logits,
                               void *scratch, size_t scratch_bytes, void *stream);

/* Launch geometry the library uses for one n x k matrix (a function of n and
 * k only, never of m). The work is cut into units of one row group (16 *
 * waves * tiles_per_wave consecutive rows) by one 256-column block; a fixed
 * number of persistent workgroups (*workgroups) each take an equal,
 * contiguous run of the *units units in row-group-major order. Also returns
 * the waves per workgroup (*waves) and 16-row tiles per wave
 * (*tiles_per_wave). Any output pointer may be NULL. Returns KQ_ERR_SHAPE for
 * invalid shapes. */
kq_status kq_launch_geometry(int64_t n, int64_t k, int *waves, int *tiles_per_wave,
                             int *workgroups, int64_t *units);

/* ------------------------------------------------- stochastic verify
 * The accept / resample rule of ch. 33 section 33.2 at temperature > 0: the
 * target judges each proposed token against its full probability row for
 * that position. The data-parallel half runs on the GPU (the probability
 * rows from the verify step's logits); the decision runs on the host, where
 * the pages keep it ("every rounding decision is visible"), in 32-bit
 * arithmetic in a fixed order. */

/* Bytes of device workspace kq_softmax_rows needs (0 for invalid shapes). */
size_t kq_softmax_workspace_bytes(int m, int64_t n);

/* Target probability rows: probs[r][j] = softmax_j(z[r]) with
 * z = l / temperature, after the optional soft cap l -> soft_cap *
 * tanh(l / soft_cap) (soft_cap = 0: none). fp32, every reduction in a fixed
 * order (deterministic).
 *  logits     device fp32 [m][n] (e.g. the verify step's logits)
 *  m, n       1 <= m <= 65535, 1 <= n < 2^31
 *  temperature > 0 and finite; soft_cap >= 0 and finite (else KQ_ERR_SHAPE)
 *  probs      device fp32 [m][n] (written; may not alias logits)
 *  workspace  device, >= kq_softmax_workspace_bytes(m, n), 256-byte aligned
 * Two launches on `stream`. */
kq_status kq_softmax_rows(const float *logits, int m, int64_t n, float temperature, float soft_cap, float *probs,
                          void *workspace, size_t workspace_bytes, void *stream);

/* The decision (host; no HIP call). k = number of proposals (0..15).
 *  draft_tokens  host int32 [k] in [0, n)
 *  draft_rows    host fp32 [k][n]: the draft's probability rows q
 *  target_rows   host fp32 [k + 1][n]: the target's rows p (kq_softmax_rows)
 *  orders        host int32 [k + 1][n]: the token order each row is walked in
 *                when it is sampled (entries in [0, n); normally a permutation)
 *  uniforms      host fp32 [k + 1] in [0, 1): u[i] decides position i; the
 *                replacement after a rejection at i uses u[i + 1], the bonus
 *                after k acceptances u[k]
 *  accepted, next_token  host int32 (written)
 * Position i is accepted when u[i] <= min(p_i[d_i] / q_i[d_i], 1) (certain
 * when q_i[d_i] <= 0). On the first rejection the replacement is drawn from
 * max(p_i - q_i, 0) divided by its fp32 sum (or from p_i when that sum is not
 * positive), walking orders[i] over the tokens with a positive residual:
 * the first token whose running fp32 sum exceeds the draw, else the last one
 * walked. After k acceptances the bonus is drawn the same way from p_k over
 * all of orders[k]. Pointers, k, n and the draft tokens are checked first;
 * the one order row that is sampled is checked whole before it is walked
 * (rows that are not sampled are not read) (KQ_ERR_NULL / SHAPE / TOKEN);
 * KQ_ERR_SHAPE also when a row to sample has no positive probability. The
 * outputs are written only on KQ_OK. */
kq_status kq_speculative_decide(int k, const int32_t *draft_tokens, int64_t n, const float *draft_rows,
                                const float *target_rows, const int32_t *orders, const float *uniforms,
                                int32_t *accepted, int32_t *next_token);

/* The same decision in two host steps, for callers that copy to the host
 * only what the decision reads: the accept tests need p_i[d_i] and
 * q_i[d_i] alone, and only the row pair of the first rejected position (or
 * target row k) is ever walked. kq_speculative_decide is exactly
 * kq_speculative_first_reject followed by kq_speculative_resample.
 *
 * kq_gather_rows (device, one launch): out[i] = rows[i][tokens[i]] for
 * i < count, e.g. p_i[d_i] from kq_softmax_rows' output.
 *  rows    device fp32 [m][n], 1 <= m <= 65535, 1 <= n < 2^31
 *  tokens  device int32 [count], 0 <= count <= m (count = 0: nothing is
 *          enqueued)
 *  out     device fp32 [count] (written); a token outside [0, n) gives a
 *          NaN, which kq_speculative_first_reject counts as a rejection */
kq_status kq_gather_rows(const float *rows, int m, int64_t n, const int32_t *tokens, int count, float *out,
                         void *stream);

/* The first rejected position: the first i < k with u[i] > min(p_at[i] /
 * q_at[i], 1) (accepted when q_at[i] <= 0; a NaN rejects), else k.
 *  p_at, q_at  host fp32 [k]: p_i[d_i] and q_i[d_i]
 *  uniforms    host fp32 [>= k]: u[0 .. k-1]
 *  position    host int32 (written)
 * KQ_ERR_NULL, KQ_ERR_SHAPE (k outside 0..15). */
kq_status kq_speculative_first_reject(int k, const float *p_at, const float *q_at, const float *uniforms,
                                      int32_t *position);

/* The token drawn where the decision stops. With q_row (a rejection): from
 * max(p_row - q_row, 0) divided by its fp32 sum in index order over the
 * tokens with a positive value, or from p_row when that sum is not positive;
 * without q_row (the bonus after k acceptances): from p_row over all of
 * `order`. The walk is kq_speculative_decide's.
 *  p_row          host fp32 [n]; q_row_or_null host fp32 [n] or NULL
 *  order          host int32 [n], entries in [0, n) (checked whole first)
 *  u              the draw: u[i + 1] after a rejection at i, u[k] for the
 *                 bonus
 *  token          host int32 (written only on KQ_OK)
 * KQ_ERR_NULL, KQ_ERR_SHAPE (n; a row with no positive value to draw),
 * KQ_ERR_TOKEN (an order entry outside [0, n)). */
kq_status kq_speculative_resample(int64_t n, const float *p_row, const float *q_row_or_null, const int32_t *order,
                                  float u, int32_t *token);

/* ------------------------------------------------- the pinned draw stream
 * The book's chapter 33, section 33.2 takes every acceptance draw and every
 * resample draw from one MT19937 stream, consumed in order; chapter 8,
 * section 8.6 (guarantee 1) requires that stream to be reimplemented bit
 * for bit and kept apart from any generic random source. This is the
 * published generator (Matsumoto and Nishimura, ACM TOMACS 8(1), 1998) with
 * its reference-code seeding, which std::mt19937 also uses: seeded with
 * 5489, its 10,000th output is 4,123,659,995.
 *
 * The float draw of one 32-bit output w is (w >> 8) * 2^-24 (fp32, exact, in
 * [0, 1 - 2^-24]); the pages do not give the conversion, so this is a
 * reading of this library.
 *
 * The state is a plain struct the caller owns (copy it to snapshot or
 * replay a stream). index is the next word to temper; 624 means the block is
 * spent and is regenerated before the next output. A state with index above
 * 624 is refused (KQ_ERR_SHAPE) and left as it is. */
#define KQ_MT19937_WORDS 624
typedef struct kq_mt19937 {
  uint32_t mt[KQ_MT19937_WORDS];
  uint32_t index;
} kq_mt19937;

/* state = the stream of `seed` (x[0] = seed, x[i] = 1812433253 (x[i-1] xor
 * (x[i-1] >> 30)) + i mod 2^32, index 624). KQ_ERR_NULL. */
kq_status kq_mt19937_seed(kq_mt19937 *state, uint32_t seed);

/* The next `count` outputs (count >= 0): 32-bit words, or float draws.
 *  out  host [count] (written); NULL allowed when count = 0
 * KQ_ERR_NULL, KQ_ERR_SHAPE (count < 0, or a corrupt state); nothing is
 * drawn on an error. */
kq_status kq_mt19937_u32(kq_mt19937 *state, uint32_t *out, int64_t count);
kq_status kq_mt19937_uniform_f32(kq_mt19937 *state, float *out, int64_t count);

/* kq_speculative_decide with its draws taken from `rng` in the pages'
 * order: the draw of each attempted proposal, then the draw of the token
 * chosen where the decision stops. rng advances by accepted + 2 draws after
 * a rejection, by k + 1 after k acceptances; the decision equals
 * kq_speculative_decide with uniforms[i] = the i-th float draw of rng.
 * Every argument check of kq_speculative_decide is made first, and on any
 * error (KQ_ERR_NULL for a null rng, KQ_ERR_SHAPE for a corrupt state) rng
 * is left unchanged and nothing is written. */
kq_status kq_speculative_decide_mt(int k, const int32_t *draft_tokens, int64_t n, const float *draft_rows,
                                   const float *target_rows, const int32_t *orders, kq_mt19937 *rng,
                                   int32_t *accepted, int32_t *next_token);

/* ---------------------------------------------------------------- chains
 * A chain launch runs a sequence of grouped products in ONE grid, each
 * phase depending on the one before it: phase i + 1 starts reading its
 * activations only after every logit of phase i is complete and visible
 * device-wide (a grid-wide barrier between phases), which is the order a
 * transformer layer imposes (q/k/v, then o, then gate/up, then down; the
 * target forward of ch. 33 section 33.1 and ch. 8 section 8.1 scores the
 * k+1 rows through all of them). Weights do not depend on earlier phases,
 * so each workgroup loads the first weights of the next phase while it
 * waits. Every phase streams its weights once for all m rows, exactly as
 * kq_gemv_staged_group does; results are within the kq.h tolerance and
 * bitwise deterministic (and bitwise equal to kq_gemv_staged_group when
 * that call uses the same geometry: 8 waves of one 16-row tile and the
 * same number of workgroups).
 *
 * Precondition: every workgroup of a chain launch is resident at once (one
 * per CU); kq_chain_encode sizes the grid from the current device's
 * capacity, assuming the chain has the device to itself while it runs.
 * Work from another stream that occupies CUs meanwhile (another chain, a
 * kernel that holds a CU) can keep workgroups from starting and the others
 * from passing a barrier. Each wait (at a barrier, or for another
 * workgroup's partial sums of a row group) is bounded: a wait longer than
 * one second gives up, sets the 32-bit word at byte KQ_CHAIN_ERROR_OFFSET of
 * the scratch to nonzero and ends the launch early (its logits are then
 * incomplete). kq_chain_status reports that word; it is sticky:
 * kq_chain_scratch_init clears it, together with the state the failed
 * launch left behind. */

#define KQ_MAX_GROUP 8
#define KQ_CHAIN_BARRIER_OFFSET 128 /* u32 arrival count of the grid barrier (zero between launches) */
#define KQ_CHAIN_ERROR_OFFSET 256   /* u32 sticky time-out word */
#define KQ_MAX_CHAIN_PHASES 65536

/* One phase: 1 <= count <= KQ_MAX_GROUP matrices of n x k (all in the
 * chain's layout, each 16-byte aligned, device) that read the same staged
 * activations (device, kq_stage_rows for this k, 256-byte aligned, staged
 * with at least the chain's m rows), each writing fp32 [m][n] logits
 * (device). */
typedef struct kq_chain_phase {
  int count;
  int64_t n, k;
  const void *w_q4k[KQ_MAX_GROUP];
  float *logits[KQ_MAX_GROUP];
  const void *staged;
} kq_chain_phase;

/* Written by kq_chain_encode, read by kq_gemv_chain (host struct). */
typedef struct kq_chain_plan {
  int32_t n_phases;
  int32_t m;
  int32_t layout;
  int32_t workgroups;     /* grid size: min(device capacity, fewest units of any phase) */
  int32_t max_groups;     /* largest number of row groups of any phase */
  int32_t tiles_per_wave; /* 16-row tiles per wave: 1 (row groups of 128 rows) */
  uint64_t table_bytes;   /* bytes of the encoded phase table */
  uint64_t scratch_bytes; /* device scratch the launch needs */
} kq_chain_plan;

/* Bytes of the encoded table of n_phases phases (0 if n_phases is out of
 * [1, KQ_MAX_CHAIN_PHASES]). */
size_t kq_chain_table_bytes(int n_phases);

/* Validate a chain and encode its phase table into table_host (host memory,
 * >= kq_chain_table_bytes(n_phases) bytes); the caller copies those bytes to
 * a device buffer (16-byte aligned) once and passes it to every
 * kq_gemv_chain call of this chain. Checks every phase as the staged calls
 * do (KQ_ERR_NULL / SHAPE / ALIGN), then queries the current device (HIP
 * calls, nothing enqueued) for how many chain workgroups it holds at once;
 * KQ_ERR_LAUNCH if that query fails. Fills *plan. The plan and table are
 * valid on the device that was current during this call. */
kq_status kq_chain_encode(const kq_chain_phase *phases, int n_phases, int m, int layout,
                          void *table_host, size_t table_bytes, kq_chain_plan *plan);

/* Initialise a chain's scratch (device, >= plan->scratch_bytes, 256-byte
 * aligned) once before its first kq_gemv_chain, and again after a launch
 * that set the error word: control words and release flags to zero, the
 * partial-sum slots to their empty pattern. Enqueued on `stream`.
 * KQ_ERR_SHAPE for a plan kq_chain_encode did not write. */
kq_status kq_chain_scratch_init(const kq_chain_plan *plan, void *scratch, size_t scratch_bytes, void *stream);

/* Run an encoded chain.
 *  table_dev  device copy of the encoded table (read only)
 *  plan       the plan kq_chain_encode wrote for it (host)
 *  scratch    device, >= plan->scratch_bytes, 256-byte aligned, initialised
 *             once by kq_chain_scratch_init; every successful launch leaves
 *             it as it found it (a timed-out one sets the error word, see
 *             above)
 * Calls sharing a scratch must be ordered (e.g. the same stream). */
kq_status kq_gemv_chain(const void *table_dev, const kq_chain_plan *plan,
                        void *scratch, size_t scratch_bytes, void *stream);

/* Outcome of the chain launches on `scratch` so far: KQ_OK, or KQ_ERR_LAUNCH
 * when a wait of one of them gave up (the time-out word is set; the logits
 * of that launch are incomplete, and the scratch needs
 * kq_chain_scratch_init before the next launch). Unlike every other call,
 * this one waits: it copies the word to the host on `stream` and
 * synchronises that stream, so it reports every launch enqueued before it.
 *  plan, scratch  as for kq_gemv_chain (the scratch of those launches)
 * KQ_ERR_NULL / SHAPE / ALIGN / WORKSPACE for invalid arguments (nothing
 * enqueued); KQ_ERR_LAUNCH also when the copy itself fails. */
kq_status kq_chain_status(const kq_chain_plan *plan, const void *scratch, size_t scratch_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
