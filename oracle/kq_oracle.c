/*
 * kq_oracle.c -- plain, slow, obviously-correct CPU oracle for the Q4_K
 * batched verify step. TEST INFRASTRUCTURE ONLY: the library under
 * quant_verify_gemv_amd/ never links, loads or calls this file; only the
 * tests, the smoke check and the bench's CPU-baseline leg do.
 *
 * What it computes (fp64 throughout):
 *
 *  1. Decode. Every Q4_K super-block is decoded to its 256 exact weights
 *     w = d * sc_j * q - dmin * m_j (sub-block j of 32 weights). The pages
 *     name the format (muser-book ch. 8 "The DFlash draft", section 8.2:
 *     draft.fc is Q4_K) and say the blocks are consumed in place, never
 *     expanded to f32 on the device (section 8.5); the byte layout is the
 *     llama.cpp GGUF one (parity against llama.cpp itself: unpinned here).
 *  2. Logits. L[m][n] = sum_k W[n][k] * x[m][k]: the target scores k+1 rows
 *     per weight read (ch. 33 "Speculation...", section 33.1; ch. 8,
 *     section 8.1). The sum runs over k in increasing order in fp64.
 *  3. Tolerance mass. A[m][n] = sum_k |W[n][k] * x[m][k]|.
 *  4. Argmax. The index of each row's largest score (ch. 8, section 8.6,
 *     guarantee 3); ties go to the lowest index. The row is "flagged" when
 *     another index j has L[i*] - L[j] <= tol[i*] + tol[j], tol = rel * A.
 *  5. Greedy accept. The temperature-0 limit of the accept/resample rule in
 *     ch. 33, section 33.2: with one-hot target and draft distributions the
 *     acceptance probability is 1 on a match and 0 on a mismatch, and the
 *     residual after a mismatch is the target's one-hot row. So accepted is
 *     the first position whose draft differs from the target argmax (or k),
 *     and next_token is the argmax of row `accepted` (the last row when all
 *     k are accepted).
 *
 * Other k-quant formats (the next formats after Q4_K: the pages say the
 * draft loads Q4_K, Q5_K and Q6_K tensors and that its v projection is
 * Q6_K, ch. 8 "The DFlash draft", section 8.2; the byte layouts are the
 * llama.cpp GGUF ones, unpinned against llama.cpp here):
 *
 *  Q5_K, 176 bytes per 256 weights: fp16 d, fp16 dmin, the same 12 bytes of
 *    6-bit scales/mins as Q4_K, 32 bytes of fifth bits, 128 bytes of
 *    nibbles. Weight i has sub-block j = i / 32, its low four bits where a
 *    Q4_K block keeps them and its fifth bit in bit j of fifth-bit byte
 *    i % 32; w = d * sc_j * q - dmin * m_j, q in [0, 31].
 *  Q6_K, 210 bytes per 256 weights: 128 bytes of low nibbles, 64 bytes of
 *    2-bit high parts, 16 signed 8-bit scales, fp16 d last. Weight i of
 *    half h = i / 128 (r = i % 128, quarter c = r / 32, l = r % 32) takes
 *    its low four bits from nibble byte 64 h + l + 32 (c & 1) (low nibble
 *    for c < 2, high for c >= 2) and its top two bits from bits 2c, 2c + 1
 *    of high-part byte 32 h + l; its scale is scale byte i / 16;
 *    w = d * sc * (q - 32), q in [0, 63].
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math, no intrinsics).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KQO_QK 256
#define KQO_BLOCK 144
#define KQO_BLOCK_Q5K 176
#define KQO_BLOCK_Q6K 210

/* Weight format codes of the *_fmt functions. */
#define KQO_Q4K 4
#define KQO_Q5K 5
#define KQO_Q6K 6

/* IEEE-754 binary16 bit pattern to double: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24). Returns NaN
 * for inf/NaN encodings so that callers can reject them. */
double kqo_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        return NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* The eight 6-bit scales and eight 6-bit mins of a super-block, from its 12
 * packed bytes. The first four of each sit in the low six bits of bytes 0-3
 * (scales) and 4-7 (mins). The last four are split: their low four bits are
 * the low/high nibble of bytes 8-11 (scales/mins) and their top two bits are
 * the spare top two bits of bytes 0-3 (scales) and 4-7 (mins). */
void kqo_scales_mins(const uint8_t *s12, int sc[8], int mn[8]) {
    for (int j = 0; j < 4; ++j) {
        sc[j] = s12[j] & 63;
        mn[j] = s12[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        int lo_sc = s12[j + 4] & 15;
        int lo_mn = s12[j + 4] >> 4;
        int hi_sc = s12[j - 4] >> 6;
        int hi_mn = s12[j] >> 6;
        sc[j] = lo_sc + 16 * hi_sc;
        mn[j] = lo_mn + 16 * hi_mn;
    }
}

/* The 4-bit quant of weight i (0..255) of a block. Weights come in four
 * groups of 64 that each own 32 bytes: the low nibbles hold the group's
 * first 32 weights, the high nibbles its second 32. */
int kqo_quant(const uint8_t *q128, int i) {
    int g = i / 64, r = i % 64;
    uint8_t b = q128[32 * g + (r % 32)];
    return r < 32 ? (b & 15) : (b >> 4);
}

/* Decode one 144-byte block into 256 exact weights. Returns 0, or -1 when
 * d or dmin is not finite. */
int kqo_decode_block(const uint8_t *blk, double *w) {
    uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t mh = (uint16_t)(blk[2] | (blk[3] << 8));
    double d = kqo_half_to_double(dh);
    double dmin = kqo_half_to_double(mh);
    if (isnan(d) || isnan(dmin)) return -1;
    int sc[8], mn[8];
    kqo_scales_mins(blk + 4, sc, mn);
    for (int i = 0; i < KQO_QK; ++i) {
        int j = i / 32;
        int q = kqo_quant(blk + 16, i);
        w[i] = d * (double)sc[j] * (double)q - dmin * (double)mn[j];
    }
    return 0;
}

/* Decode a full row of K weights. */
int kqo_decode_row(const uint8_t *row, int64_t k, double *w) {
    for (int64_t b = 0; b < k / KQO_QK; ++b)
        if (kqo_decode_block(row + b * KQO_BLOCK, w + b * KQO_QK)) return -1;
    return 0;
}

/* The 5-bit quant of weight i of a Q5_K block: four low bits from the
 * nibbles (as in Q4_K), the fifth from bit i / 32 of byte i % 32 of qh. */
int kqo_quant_q5k(const uint8_t *qh32, const uint8_t *q128, int i) {
    int hi = (qh32[i % 32] >> (i / 32)) & 1;
    return kqo_quant(q128, i) + 16 * hi;
}

/* Decode one 176-byte Q5_K block; 0, or -1 when d or dmin is not finite. */
int kqo_decode_block_q5k(const uint8_t *blk, double *w) {
    uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t mh = (uint16_t)(blk[2] | (blk[3] << 8));
    double d = kqo_half_to_double(dh);
    double dmin = kqo_half_to_double(mh);
    if (isnan(d) || isnan(dmin)) return -1;
    int sc[8], mn[8];
    kqo_scales_mins(blk + 4, sc, mn);
    for (int i = 0; i < KQO_QK; ++i) {
        int j = i / 32;
        int q = kqo_quant_q5k(blk + 16, blk + 48, i);
        w[i] = d * (double)sc[j] * (double)q - dmin * (double)mn[j];
    }
    return 0;
}

/* The 6-bit quant (0..63, before the -32 offset) of weight i of a Q6_K
 * block from its 128 nibble bytes and 64 high-part bytes. */
int kqo_quant_q6k(const uint8_t *ql, const uint8_t *qh, int i) {
    int h = i / 128, r = i % 128, c = r / 32, l = r % 32;
    uint8_t b = ql[64 * h + l + 32 * (c & 1)];
    int lo = c < 2 ? (b & 15) : (b >> 4);
    int hi = (qh[32 * h + l] >> (2 * c)) & 3;
    return lo | (hi << 4);
}

/* Decode one 210-byte Q6_K block; 0, or -1 when d is not finite. */
int kqo_decode_block_q6k(const uint8_t *blk, double *w) {
    const uint8_t *ql = blk, *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    uint16_t dh = (uint16_t)(blk[208] | (blk[209] << 8));
    double d = kqo_half_to_double(dh);
    if (isnan(d)) return -1;
    for (int i = 0; i < KQO_QK; ++i)
        w[i] = d * (double)sc[i / 16] * (double)(kqo_quant_q6k(ql, qh, i) - 32);
    return 0;
}

/* Bytes per 256-weight block of a format code (0 for an unknown code). */
int kqo_block_bytes(int fmt) {
    return fmt == KQO_Q4K ? KQO_BLOCK : fmt == KQO_Q5K ? KQO_BLOCK_Q5K : fmt == KQO_Q6K ? KQO_BLOCK_Q6K : 0;
}

/* Decode one block of format `fmt`; -1 for a non-finite header, -4 for an
 * unknown format. */
int kqo_decode_block_fmt(int fmt, const uint8_t *blk, double *w) {
    if (fmt == KQO_Q4K) return kqo_decode_block(blk, w);
    if (fmt == KQO_Q5K) return kqo_decode_block_q5k(blk, w);
    if (fmt == KQO_Q6K) return kqo_decode_block_q6k(blk, w);
    return -4;
}

/* Decode a full row of K weights of format `fmt`. */
int kqo_decode_row_fmt(int fmt, const uint8_t *row, int64_t k, double *w) {
    int bb = kqo_block_bytes(fmt);
    if (!bb) return -4;
    for (int64_t b = 0; b < k / KQO_QK; ++b) {
        int rc = kqo_decode_block_fmt(fmt, row + b * bb, w + b * KQO_QK);
        if (rc) return rc;
    }
    return 0;
}

/* L[m][n] and A[m][n] (row-major [m][n], fp64) for an N x K Q4_K matrix and
 * M fp32 activation rows [m][k]. `rows` may be NULL (all rows 0..n-1) or a
 * list of n_rows row indices, in which case outputs are [m][n_rows].
 * Returns 0; -1 for bad shapes; -2 for a non-finite d/dmin; -3 for a
 * non-finite activation. nthreads <= 0 keeps the OpenMP default. */
int kqo_gemv_rows_fmt(int fmt, const uint8_t *w, int64_t n, int64_t k, const float *x, int m,
                      const int64_t *rows, int64_t n_rows, double *L, double *A,
                      int nthreads);

int kqo_gemv_rows(const uint8_t *w, int64_t n, int64_t k, const float *x, int m,
                  const int64_t *rows, int64_t n_rows, double *L, double *A,
                  int nthreads) {
    return kqo_gemv_rows_fmt(KQO_Q4K, w, n, k, x, m, rows, n_rows, L, A, nthreads);
}

/* kqo_gemv_rows for a matrix in format `fmt` (rows of K / 256 blocks of
 * kqo_block_bytes(fmt) bytes); -4 for an unknown format. */
int kqo_gemv_rows_fmt(int fmt, const uint8_t *w, int64_t n, int64_t k, const float *x, int m,
                      const int64_t *rows, int64_t n_rows, double *L, double *A,
                      int nthreads) {
    if (!kqo_block_bytes(fmt)) return -4;
    if (n <= 0 || k <= 0 || k % KQO_QK || m <= 0) return -1;
    for (int64_t i = 0; i < (int64_t)m * k; ++i)
        if (!isfinite(x[i])) return -3;
    int64_t nout = rows ? n_rows : n;
    for (int64_t r = 0; r < nout; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n)) return -1;
    int64_t row_bytes = (k / KQO_QK) * kqo_block_bytes(fmt);
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *wr = (double *)malloc(sizeof(double) * (size_t)k);
        double *s = (double *)malloc(sizeof(double) * (size_t)m);
        double *a = (double *)malloc(sizeof(double) * (size_t)m);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nout; ++r) {
            int64_t nn = rows ? rows[r] : r;
            if (kqo_decode_row_fmt(fmt, w + nn * row_bytes, k, wr)) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int mm = 0; mm < m; ++mm) { s[mm] = 0.0; a[mm] = 0.0; }
            for (int64_t kk = 0; kk < k; ++kk) {
                for (int mm = 0; mm < m; ++mm) {
                    double p = wr[kk] * (double)x[(int64_t)mm * k + kk];
                    s[mm] += p;
                    a[mm] += fabs(p);
                }
            }
            for (int mm = 0; mm < m; ++mm) {
                L[(int64_t)mm * nout + r] = s[mm];
                A[(int64_t)mm * nout + r] = a[mm];
            }
        }
        free(wr); free(s); free(a);
    }
    return bad ? -2 : 0;
}

/* Mass of the two terms of each Q4_K weight: B[m][n] = sum_k (|d sc_j q_k|
 * + |dmin m_j|) |x[m][k]|, where w_k = d sc_j q_k - dmin m_j (the same
 * decode as kqo_decode_block, its two terms kept apart). This is not part
 * of what the method computes. It is the quantity a kernel that forms the
 * scale term and the min term of a block separately (each from exact
 * products) and subtracts them in floating point has its rounding error
 * proportional to; B >= A, with equality when no weight mixes a positive
 * scale term with a positive min term (dmin = 0, or q = 0 everywhere).
 * Outputs [m][n_rows] (rows may be NULL: all n rows); returns as
 * kqo_gemv_rows. */
int kqo_term_mass_q4k(const uint8_t *w, int64_t n, int64_t k, const float *x, int m,
                      const int64_t *rows, int64_t n_rows, double *B) {
    if (n <= 0 || k <= 0 || k % KQO_QK || m <= 0) return -1;
    for (int64_t i = 0; i < (int64_t)m * k; ++i)
        if (!isfinite(x[i])) return -3;
    int64_t nout = rows ? n_rows : n;
    for (int64_t r = 0; r < nout; ++r)
        if (rows && (rows[r] < 0 || rows[r] >= n)) return -1;
    int64_t row_bytes = (k / KQO_QK) * KQO_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nout; ++r) {
        int64_t nn = rows ? rows[r] : r;
        for (int mm = 0; mm < m; ++mm) B[(int64_t)mm * nout + r] = 0.0;
        for (int64_t b = 0; b < k / KQO_QK; ++b) {
            const uint8_t *blk = w + nn * row_bytes + b * KQO_BLOCK;
            double d = kqo_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
            double dmin = kqo_half_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
            if (isnan(d) || isnan(dmin)) {
#pragma omp atomic write
                bad = 1;
                break;
            }
            int sc[8], mn[8];
            kqo_scales_mins(blk + 4, sc, mn);
            for (int i = 0; i < KQO_QK; ++i) {
                int j = i / 32;
                double term = fabs(d * (double)sc[j] * (double)kqo_quant(blk + 16, i)) +
                              fabs(dmin * (double)mn[j]);
                int64_t kk = b * KQO_QK + i;
                for (int mm = 0; mm < m; ++mm)
                    B[(int64_t)mm * nout + r] += term * fabs((double)x[(int64_t)mm * k + kk]);
            }
        }
    }
    return bad ? -2 : 0;
}

/* Per row m: argmax[m] = lowest index attaining the maximum of L[m][:],
 * n_cand[m] = number of other indices j with
 * L[i*] - L[j] <= rel * (A[i*] + A[j]) (0 means the row is unflagged). */
int kqo_argmax_flags(const double *L, const double *A, int m, int64_t n,
                     double rel, int32_t *argmax, int64_t *n_cand) {
    if (m <= 0 || n <= 0) return -1;
    for (int mm = 0; mm < m; ++mm) {
        const double *l = L + (int64_t)mm * n;
        const double *a = A + (int64_t)mm * n;
        int64_t best = 0;
        for (int64_t j = 1; j < n; ++j)
            if (l[j] > l[best]) best = j;
        int64_t c = 0;
        for (int64_t j = 0; j < n; ++j)
            if (j != best && l[best] - l[j] <= rel * (a[best] + a[j])) ++c;
        argmax[mm] = (int32_t)best;
        n_cand[mm] = c;
    }
    return 0;
}

/* Candidate set of row m (the indices counted by kqo_argmax_flags), written
 * in increasing order to out[0..cap); returns how many exist. */
int64_t kqo_candidates(const double *L, const double *A, int64_t n, int32_t best,
                       double rel, int32_t *out, int64_t cap) {
    int64_t c = 0;
    for (int64_t j = 0; j < n; ++j) {
        if (j == best) continue;
        if (L[best] - L[j] <= rel * (A[best] + A[j])) {
            if (c < cap) out[c] = (int32_t)j;
            ++c;
        }
    }
    return c;
}

/* Greedy accept over k draft tokens judged by rows 0..k of the target.
 * Row i < k judges draft[i]; row k supplies the bonus token. */
int kqo_accept(const int32_t *draft, int k, const int32_t *argmax,
               int32_t *accepted, int32_t *next_token) {
    if (k < 0) return -1;
    int i = 0;
    while (i < k && draft[i] == argmax[i]) ++i;
    *accepted = i;
    *next_token = argmax[i];
    return 0;
}

/* Greedy accept over a token tree of m nodes (the hardware-aware token tree
 * of ch. 33 "Speculation: the local win and the distributed verdict",
 * section 33.7: the tree covers near-miss branches with batch arithmetic
 * the weight stream leaves idle, so the target scores every node in one
 * pass and a round emits along the branch it agrees with). Node 0 is the
 * root (the last committed position); node j >= 1 proposes token[j] as
 * the continuation of its parent parent[j] < j. Row j of the target
 * predicts the token after node j (its argmax). From the root, the walk
 * moves to a child whose token equals the current node's argmax (the
 * lowest-index such child when siblings repeat a token) and stops when no
 * child matches. accepted = nodes moved through, next_token = the argmax of
 * the node where the walk stops, path[0..accepted) = the nodes moved
 * through. A chain (parent[j] = j - 1) is the linear rule of kqo_accept.
 * Returns -1 for an invalid tree (parent[0] != -1 or parent[j] not in
 * [0, j)). */
int kqo_tree_accept(const int32_t *parent, const int32_t *token, int m, const int32_t *argmax,
                    int32_t *accepted, int32_t *next_token, int32_t *path) {
    if (m < 1 || parent[0] != -1) return -1;
    for (int j = 1; j < m; ++j)
        if (parent[j] < 0 || parent[j] >= j) return -1;
    int cur = 0, n = 0;
    for (;;) {
        int nxt = -1;
        for (int j = 1; j < m; ++j)
            if (parent[j] == cur && token[j] == argmax[cur]) { nxt = j; break; }
        if (nxt < 0) break;
        path[n++] = nxt;
        cur = nxt;
    }
    *accepted = n;
    *next_token = argmax[cur];
    return 0;
}

int kqo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
