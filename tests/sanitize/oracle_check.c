/* Driver of the CPU sanitizer build of the oracle (oracle/kq_oracle.c, built
 * by gcc with -fsanitize=address,undefined and no recovery, with OpenMP). It
 * runs every oracle function on random and edge inputs -- all 65,536 half
 * patterns, random blocks of the three formats (including non-finite
 * headers), products on full and sampled rows at 1 and 4 threads, argmax
 * flags and candidate lists with short buffers, linear and tree accepts
 * including refused trees -- and checks the relations that hold between
 * them. Prints one line and exits 0 when every expectation holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double kqo_half_to_double(uint16_t h);
void kqo_scales_mins(const uint8_t *s12, int sc[8], int mn[8]);
int kqo_block_bytes(int fmt);
int kqo_decode_block_fmt(int fmt, const uint8_t *blk, double *w);
int kqo_decode_row_fmt(int fmt, const uint8_t *row, int64_t k, double *w);
int kqo_gemv_rows_fmt(int fmt, const uint8_t *w, int64_t n, int64_t k, const float *x, int m, const int64_t *rows,
                      int64_t n_rows, double *L, double *A, int nthreads);
int kqo_term_mass_q4k(const uint8_t *w, int64_t n, int64_t k, const float *x, int m, const int64_t *rows,
                      int64_t n_rows, double *B);
int kqo_argmax_flags(const double *L, const double *A, int m, int64_t n, double rel, int32_t *argmax,
                     int64_t *n_cand);
int64_t kqo_candidates(const double *L, const double *A, int64_t n, int32_t best, double rel, int32_t *out,
                       int64_t cap);
int kqo_accept(const int32_t *draft, int k, const int32_t *argmax, int32_t *accepted, int32_t *next_token);
int kqo_tree_accept(const int32_t *parent, const int32_t *token, int m, const int32_t *argmax, int32_t *accepted,
                    int32_t *next_token, int32_t *path);

/* the oracle's format codes */
enum { FMT_Q4K = 4, FMT_Q5K = 5, FMT_Q6K = 6 };

static int checks = 0, failed = 0;
#define EXPECT(c)                                                            \
    do {                                                                     \
        ++checks;                                                            \
        if (!(c)) {                                                          \
            ++failed;                                                        \
            fprintf(stderr, "oracle_check: line %d: %s\n", __LINE__, #c);   \
        }                                                                    \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 2685821657736338717ull) >> 32);
}
static float gauss(void) {
    double u = (rnd() + 1.0) / 4294967297.0, v = rnd() / 4294967296.0;
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static uint16_t half_bits(double v) { /* a normal fp16 near v > 0 (truncated) */
    int e = 0;
    double f = frexp(v, &e); /* v = f 2^e, f in [0.5, 1) */
    return (uint16_t)(((e - 1 + 15) << 10) | ((int)((f * 2.0 - 1.0) * 1024.0) & 0x3FF));
}

/* random matrix of `fmt`: random bytes with a finite positive small d (and
 * dmin) in every block */
static void random_matrix(int fmt, uint8_t *w, int64_t n, int64_t k) {
    const int bb = kqo_block_bytes(fmt);
    for (int64_t b = 0; b < n * (k / 256); ++b) {
        uint8_t *blk = w + b * bb;
        for (int i = 0; i < bb; ++i) blk[i] = (uint8_t)rnd();
        const uint16_t d = half_bits(0.001 + 0.049 * (rnd() / 4294967296.0));
        const uint16_t dm = half_bits(0.001 + 0.049 * (rnd() / 4294967296.0));
        if (fmt == FMT_Q6K) {
            blk[208] = (uint8_t)d;
            blk[209] = (uint8_t)(d >> 8);
        } else {
            blk[0] = (uint8_t)d;
            blk[1] = (uint8_t)(d >> 8);
            blk[2] = (uint8_t)dm;
            blk[3] = (uint8_t)(dm >> 8);
        }
    }
}

static void halves_and_blocks(void) {
    for (uint32_t h = 0; h < 65536; ++h) {
        const double v = kqo_half_to_double((uint16_t)h);
        const uint32_t e = (h >> 10) & 31;
        EXPECT((e == 31) == !isfinite(v));
    }
    uint8_t blk[256];
    double w[256];
    int sc[8], mn[8];
    for (int t = 0; t < 2000; ++t) {
        for (int i = 0; i < 256; ++i) blk[i] = (uint8_t)rnd();
        kqo_scales_mins(blk + 4, sc, mn);
        for (int j = 0; j < 8; ++j) EXPECT(sc[j] >= 0 && sc[j] < 64 && mn[j] >= 0 && mn[j] < 64);
        for (int fmt = FMT_Q4K; fmt <= FMT_Q6K; ++fmt) {
            const int r = kqo_decode_block_fmt(fmt, blk, w);
            EXPECT(r == 0 || r == -1); /* -1: an inf or NaN header */
        }
    }
    EXPECT(kqo_block_bytes(FMT_Q4K) == 144 && kqo_block_bytes(FMT_Q5K) == 176 && kqo_block_bytes(FMT_Q6K) == 210);
    EXPECT(kqo_block_bytes(3) == 0 && kqo_block_bytes(7) == 0);
    EXPECT(kqo_decode_block_fmt(3, blk, w) == -4);
}

static void products(int nthreads) {
    const int64_t n = 37, k = 768;
    const int m = 5;
    for (int fmt = FMT_Q4K; fmt <= FMT_Q6K; ++fmt) {
        const int bb = kqo_block_bytes(fmt);
        uint8_t *w = malloc((size_t)(n * (k / 256) * bb));
        float *x = malloc(sizeof(float) * m * k);
        double *L = malloc(sizeof(double) * m * n), *A = malloc(sizeof(double) * m * n);
        double *Ls = malloc(sizeof(double) * m * 4), *As = malloc(sizeof(double) * m * 4);
        random_matrix(fmt, w, n, k);
        for (int i = 0; i < m * k; ++i) x[i] = gauss();
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k, x, m, NULL, 0, L, A, nthreads) == 0);
        for (int i = 0; i < m * n; ++i) EXPECT(A[i] >= fabs(L[i]));
        const int64_t rows[4] = {36, 0, 17, 36};
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k, x, m, rows, 4, Ls, As, nthreads) == 0);
        for (int mm = 0; mm < m; ++mm)
            for (int r = 0; r < 4; ++r)
                EXPECT(Ls[mm * 4 + r] == L[mm * n + rows[r]] && As[mm * 4 + r] == A[mm * n + rows[r]]);
        if (fmt == FMT_Q4K) {
            double *B = malloc(sizeof(double) * m * n);
            EXPECT(kqo_term_mass_q4k(w, n, k, x, m, NULL, 0, B) == 0);
            for (int i = 0; i < m * n; ++i) EXPECT(B[i] >= A[i] * (1 - 1e-12));
            const int64_t bad_rows[1] = {n};
            EXPECT(kqo_term_mass_q4k(w, n, k, x, m, bad_rows, 1, B) == -1);
            free(B);
        }
        /* refusals: bad rows, shapes, non-finite input, unknown format */
        const int64_t bad[2] = {0, n};
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k, x, m, bad, 2, Ls, As, nthreads) == -1);
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k + 1, x, m, NULL, 0, L, A, nthreads) == -1);
        EXPECT(kqo_gemv_rows_fmt(3, w, n, k, x, m, NULL, 0, L, A, nthreads) == -4);
        x[3] = NAN;
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k, x, m, NULL, 0, L, A, nthreads) == -3);
        x[3] = 0.5f;
        if (fmt == FMT_Q6K) {
            w[208] = 0x00;
            w[209] = 0x7C; /* +inf d in the first block */
        } else {
            w[0] = 0x00;
            w[1] = 0x7C;
        }
        EXPECT(kqo_gemv_rows_fmt(fmt, w, n, k, x, m, NULL, 0, L, A, nthreads) == -2);
        free(w); free(x); free(L); free(A); free(Ls); free(As);
    }
}

static void decisions(void) {
    const int m = 3;
    const int64_t n = 200;
    double L[600], A[600];
    int32_t am[3], out[8];
    int64_t nc[3];
    for (int t = 0; t < 300; ++t) {
        for (int i = 0; i < m * n; ++i) {
            L[i] = (double)(rnd() % 50) * 0.25;
            A[i] = 1.0 + rnd() % 100;
        }
        EXPECT(kqo_argmax_flags(L, A, m, n, 1e-3, am, nc) == 0);
        for (int r = 0; r < m; ++r) {
            const int64_t c = kqo_candidates(L + r * n, A + r * n, n, am[r], 1e-3, out, 8);
            EXPECT(c == nc[r]);
            for (int64_t j = 0; j < n; ++j) EXPECT(L[r * n + j] <= L[r * n + am[r]]);
        }
    }
    EXPECT(kqo_argmax_flags(L, A, 0, n, 1e-3, am, nc) == -1);
    int32_t draft[16], argmax[17], acc = -1, nxt = -1;
    for (int t = 0; t < 500; ++t) {
        const int k = (int)(rnd() % 16);
        for (int i = 0; i <= k; ++i) argmax[i] = (int32_t)(rnd() % 4);
        for (int i = 0; i < k; ++i) draft[i] = (int32_t)(rnd() % 4);
        EXPECT(kqo_accept(draft, k, argmax, &acc, &nxt) == 0);
        EXPECT(acc >= 0 && acc <= k && nxt == argmax[acc]);
    }
    int32_t parent[64], token[64], path[64];
    for (int t = 0; t < 500; ++t) {
        const int mm = 1 + (int)(rnd() % 64);
        parent[0] = -1;
        for (int j = 1; j < mm; ++j) {
            parent[j] = (int32_t)(rnd() % j);
            token[j] = (int32_t)(rnd() % 3);
        }
        int32_t amx[64];
        for (int j = 0; j < mm; ++j) amx[j] = (int32_t)(rnd() % 3);
        EXPECT(kqo_tree_accept(parent, token, mm, amx, &acc, &nxt, path) == 0);
        EXPECT(acc >= 0 && acc < mm);
        int cur = 0;
        for (int s = 0; s < acc; ++s) {
            EXPECT(parent[path[s]] == cur && token[path[s]] == amx[cur]);
            cur = path[s];
        }
        EXPECT(nxt == amx[cur]);
        if (mm > 1) {
            const int j = 1 + (int)(rnd() % (mm - 1));
            parent[j] = j;
            EXPECT(kqo_tree_accept(parent, token, mm, amx, &acc, &nxt, path) == -1);
        }
    }
}

int main(void) {
    halves_and_blocks();
    products(1);
    products(4);
    decisions();
    printf("oracle_check: %d checks, %d failed\n", checks, failed);
    return failed ? 1 : 0;
}
