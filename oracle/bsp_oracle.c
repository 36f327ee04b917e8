/*
 * bsp_oracle.c -- plain, slow CPU oracle for the bitmap-tiled sparse matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or table with the HIP path.
 *
 * What it computes (sources are the three pages the method is described on):
 *
 *  - Encoding, from UnionSparse (IEEE TCAD), Sec. V-A "IE-BME Representation",
 *    paragraphs "Union Bitmaps", "Union Value Offsets" and "Compressed
 *    Values", taken with a single area per tile (R_A = C_A = 1, so Q = 1) on a
 *    1 x 64 tile: the union mask is then the plain nonzero mask, the tile
 *    offset is the prefix sum of the preceding tiles' popcounts, and value
 *    (i,j) of tile t is stored at CV[o_t + rho_t(i,j)], with rho the number of
 *    active positions before (i,j).
 *  - Bit order: the first (leftmost) column of a tile is the least
 *    significant bit of its word (same paragraph, worked example of Fig. 7).
 *  - The product: Y = W_sparse * X (SPDP, Sec. 2.2 problem statement; the
 *    UnionSparse SpMM of Sec. VI). With int4 weights and activations the
 *    exact result is an integer sum; it is computed here in int64 and must
 *    fit int32. For fp16 operands the reference is the exact-product fp64
 *    sum (fp16 x fp16 products are exact in fp64).
 *
 * Readings where the pages leave a detail open (each is also listed in the
 * design notes):
 *  - tiles run over the matrix in row-major order, g = m*T + t, T = ceil(K/64);
 *  - offsets are uint32 element counts with G+1 entries, offsets[G] = nnz;
 *  - int4 payload element e sits in byte e>>1, low nibble when e is even,
 *    as a 4-bit two's-complement code; an odd count leaves the last high
 *    nibble zero; there is no padding;
 *  - a last partial tile (K % 64 != 0) has zero bits for columns >= K;
 *  - a position is active iff its value is nonzero (fp16: +0 and -0 are
 *    zero, NaN is nonzero);
 *  - X is the K x N matrix stored column by column, i.e. an [N][K] array;
 *    int4 X is packed along K two per byte, low nibble = even k, row stride
 *    ceil(K/2) bytes; fp16 X rows are K elements;
 *  - Y is an [N][M] array (M x N stored column by column).
 *
 * Every function is a direct transcription of a definition; no blocking, no
 * reordering, no tricks.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>
#include <math.h>
#include <pthread.h>

#define OR_OK 0
#define OR_E_ARG 1
#define OR_E_RANGE 2
#define OR_E_CAPACITY 3
#define OR_E_OVERFLOW 4

/* Number of 1 x 64 tiles covering a row of K columns. */
int64_t or_tiles_per_row(int64_t K) { return (K + 63) / 64; }

/* Count of set bits, one bit at a time. */
int or_popcount64(uint64_t w) {
    int c = 0;
    for (int j = 0; j < 64; ++j)
        if ((w >> j) & 1u) c++;
    return c;
}

/* rho: number of active positions strictly before position j of a tile word. */
int or_rank(uint64_t w, int j) {
    int c = 0;
    for (int i = 0; i < j; ++i)
        if ((w >> i) & 1u) c++;
    return c;
}

/* Store / fetch int4 payload element e (4-bit two's complement). */
static void put_nibble(uint8_t *payload, int64_t e, int v) {
    uint8_t code = (uint8_t)(v & 0xF);
    if (e % 2 == 0) payload[e / 2] = (uint8_t)((payload[e / 2] & 0xF0) | code);
    else            payload[e / 2] = (uint8_t)((payload[e / 2] & 0x0F) | (code << 4));
}

static int get_nibble(const uint8_t *payload, int64_t e) {
    int code = (e % 2 == 0) ? (payload[e / 2] & 0xF) : (payload[e / 2] >> 4);
    return code >= 8 ? code - 16 : code;
}

/* fp16 zero test: +0 (0x0000) and -0 (0x8000) are zero, everything else
 * (subnormals, inf, NaN) is a stored value. */
static int f16_is_zero(uint16_t h) { return (h & 0x7FFF) == 0; }

/* IEEE 754 binary16 -> double, from the format's definition:
 * sign bit, 5-bit biased exponent (bias 15), 10-bit fraction. */
double or_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0)        v = ldexp((double)frac, -24);          /* subnormal: frac * 2^-14 * 2^-10 */
    else if (expo == 31)  v = frac ? NAN : INFINITY;
    else                  v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

/*
 * Reference encoder. dtype 0: W is int8 holding values in [-8, 7];
 * dtype 1: W holds IEEE binary16 bit patterns. Row-major with leading
 * dimension ldw. Outputs: bitmaps[M*T], offsets[M*T+1], payload.
 * payload_cap is in bytes. Any output pointer may be NULL (then only the
 * counts are produced). Returns OR_* codes; nnz_out and bytes_out are written
 * whenever the input is valid.
 */
int or_encode(int dtype, const void *W, int64_t M, int64_t K, int64_t ldw,
              uint64_t *bitmaps, uint32_t *offsets, void *payload, int64_t payload_cap,
              int64_t *nnz_out, int64_t *bytes_out) {
    if (M < 0 || K < 0 || ldw < K || (dtype != 0 && dtype != 1)) return OR_E_ARG;
    if (W == NULL && M > 0 && K > 0) return OR_E_ARG;
    const int8_t *Wi = (const int8_t *)W;
    const uint16_t *Wh = (const uint16_t *)W;
    int64_t T = or_tiles_per_row(K);

    /* Pass 1: validate values and count nonzeros. */
    int64_t nnz = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            if (dtype == 0) {
                int v = Wi[m * ldw + k];
                if (v < -8 || v > 7) return OR_E_RANGE;
                if (v != 0) nnz++;
            } else {
                if (!f16_is_zero(Wh[m * ldw + k])) nnz++;
            }
        }
    if (nnz > (int64_t)UINT32_MAX) return OR_E_OVERFLOW;
    int64_t bytes = (dtype == 0) ? (nnz + 1) / 2 : 2 * nnz;
    if (nnz_out) *nnz_out = nnz;
    if (bytes_out) *bytes_out = bytes;
    if (payload != NULL && payload_cap < bytes) return OR_E_CAPACITY;

    /* Pass 2: one word, one offset and the tile's values, tile by tile. */
    if (payload != NULL && dtype == 0 && bytes > 0) memset(payload, 0, (size_t)bytes);
    int64_t off = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t t = 0; t < T; ++t) {
            int64_t g = m * T + t;
            uint64_t word = 0;
            if (offsets) offsets[g] = (uint32_t)off;
            for (int j = 0; j < 64; ++j) {
                int64_t k = 64 * t + j;
                if (k >= K) break;
                int nonzero = (dtype == 0) ? (Wi[m * ldw + k] != 0) : !f16_is_zero(Wh[m * ldw + k]);
                if (!nonzero) continue;
                word |= (uint64_t)1 << j;
                if (payload != NULL) {
                    if (dtype == 0) put_nibble((uint8_t *)payload, off, Wi[m * ldw + k]);
                    else            ((uint16_t *)payload)[off] = Wh[m * ldw + k];
                }
                off++;
            }
            if (bitmaps) bitmaps[g] = word;
        }
    if (offsets) offsets[M * T] = (uint32_t)off;
    return OR_OK;
}

/*
 * Stream validator. Returns 0 when every invariant holds, otherwise the
 * number of the first one that fails:
 *  1 offsets[0] != 0
 *  2 offsets[g+1] - offsets[g] != popcount(bitmaps[g]) for some g
 *  3 payload size: bytes != ceil(nnz/2) (int4) or 2*nnz (fp16)
 *  4 a bit is set at a column >= K in a last tile
 *  5 an int4 odd count whose final high nibble is not zero
 *  6 a stored value that is zero (int4 code 0, or fp16 +-0)
 */
int or_validate(int dtype, const uint64_t *bitmaps, const uint32_t *offsets,
                const void *payload, int64_t payload_bytes, int64_t M, int64_t K) {
    int64_t T = or_tiles_per_row(K);
    int64_t G = M * T;
    if (offsets[0] != 0) return 1;
    for (int64_t g = 0; g < G; ++g)
        if ((int64_t)offsets[g + 1] - (int64_t)offsets[g] != or_popcount64(bitmaps[g])) return 2;
    int64_t nnz = offsets[G];
    int64_t want = (dtype == 0) ? (nnz + 1) / 2 : 2 * nnz;
    if (payload_bytes != want) return 3;
    if (K % 64 != 0)
        for (int64_t m = 0; m < M; ++m) {
            uint64_t w = bitmaps[m * T + T - 1];
            for (int j = (int)(K % 64); j < 64; ++j)
                if ((w >> j) & 1u) return 4;
        }
    if (dtype == 0) {
        const uint8_t *p = (const uint8_t *)payload;
        if (nnz % 2 == 1 && (p[nnz / 2] >> 4) != 0) return 5;
        for (int64_t e = 0; e < nnz; ++e)
            if (get_nibble(p, e) == 0) return 6;
    } else {
        const uint16_t *p = (const uint16_t *)payload;
        for (int64_t e = 0; e < nnz; ++e)
            if (f16_is_zero(p[e])) return 6;
    }
    return 0;
}

/* Decode to a dense row-major M x K array (int8 values, or fp16 bit patterns):
 * W[m, 64t+j] = bit j of word g ? CV[offsets[g] + rho(word, j)] : 0. */
void or_decode(int dtype, const uint64_t *bitmaps, const uint32_t *offsets,
               const void *payload, int64_t M, int64_t K, void *Wd) {
    int64_t T = or_tiles_per_row(K);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            int64_t t = k / 64;
            int j = (int)(k % 64);
            int64_t g = m * T + t;
            uint64_t word = bitmaps[g];
            int bit = (int)((word >> j) & 1u);
            int64_t e = (int64_t)offsets[g] + or_rank(word, j);
            if (dtype == 0)
                ((int8_t *)Wd)[m * K + k] = bit ? (int8_t)get_nibble((const uint8_t *)payload, e) : 0;
            else
                ((uint16_t *)Wd)[m * K + k] = bit ? ((const uint16_t *)payload)[e] : 0;
        }
}

/* Unpack int4 activations: X[n][k] = nibble k of row n (row stride ceil(K/2) bytes). */
void or_unpack_x4(const uint8_t *Xp, int64_t N, int64_t K, int8_t *Xd) {
    int64_t stride = (K + 1) / 2;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            Xd[n * K + k] = (int8_t)get_nibble(Xp + n * stride, k);
}

/* Exact integer product: Y[n][m] = sum_k W[m][k] * X[n][k] in int64. */
void or_matmul_i64(const int8_t *Wd, int64_t M, int64_t K, const int8_t *Xd, int64_t N, int64_t *Y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)Wd[m * K + k] * (int64_t)Xd[n * K + k];
            Y[n * M + m] = acc;
        }
}

/* fp64 reference product of fp16 operands (products are exact in fp64). */
void or_matmul_f64(const uint16_t *Wd, int64_t M, int64_t K, const uint16_t *Xh, int64_t N, double *Y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += or_f16_to_f64(Wd[m * K + k]) * or_f16_to_f64(Xh[n * K + k]);
            Y[n * M + m] = acc;
        }
}

/*
 * The whole int4 path: decode the stream, unpack X, exact product, then the
 * int32 result. Returns OR_E_OVERFLOW if a sum does not fit int32.
 */
int or_spmm_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                 int64_t M, int64_t K, const uint8_t *Xp, int64_t N, int32_t *Y) {
    int8_t *Wd = (int8_t *)malloc((size_t)(M * K > 0 ? M * K : 1));
    int8_t *Xd = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
    int64_t *Y64 = (int64_t *)malloc((size_t)(M * N > 0 ? M * N : 1) * sizeof(int64_t));
    if (!Wd || !Xd || !Y64) { free(Wd); free(Xd); free(Y64); return OR_E_ARG; }
    or_decode(0, bitmaps, offsets, payload, M, K, Wd);
    or_unpack_x4(Xp, N, K, Xd);
    or_matmul_i64(Wd, M, K, Xd, N, Y64);
    int rc = OR_OK;
    for (int64_t i = 0; i < M * N; ++i) {
        if (Y64[i] > INT32_MAX || Y64[i] < INT32_MIN) rc = OR_E_OVERFLOW;
        Y[i] = (int32_t)Y64[i];
    }
    free(Wd); free(Xd); free(Y64);
    return rc;
}

/* The whole fp16 path, as the fp64 reference r[n][m]. */
int or_spmm_f16(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                int64_t M, int64_t K, const uint16_t *Xh, int64_t N, double *Y) {
    uint16_t *Wd = (uint16_t *)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(uint16_t));
    if (!Wd) return OR_E_ARG;
    or_decode(1, bitmaps, offsets, payload, M, K, Wd);
    or_matmul_f64(Wd, M, K, Xh, N, Y);
    free(Wd);
    return OR_OK;
}

/* Single output sample: Y[n][m] computed straight from the stream, for
 * spot-checking very large problems one element at a time. */
int64_t or_spmm_w4a4_one(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                         int64_t K, const uint8_t *Xp, int64_t m, int64_t n) {
    int64_t T = or_tiles_per_row(K);
    int64_t stride = (K + 1) / 2;
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = m * T + k / 64;
        int j = (int)(k % 64);
        uint64_t word = bitmaps[g];
        if (!((word >> j) & 1u)) continue;
        int w = get_nibble(payload, (int64_t)offsets[g] + or_rank(word, j));
        int x = get_nibble(Xp + n * stride, k);
        acc += (int64_t)w * x;
    }
    return acc;
}

double or_spmm_f16_one(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                       int64_t K, const uint16_t *Xh, int64_t m, int64_t n) {
    int64_t T = or_tiles_per_row(K);
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = m * T + k / 64;
        int j = (int)(k % 64);
        uint64_t word = bitmaps[g];
        if (!((word >> j) & 1u)) continue;
        uint16_t w = payload[(int64_t)offsets[g] + or_rank(word, j)];
        acc += or_f16_to_f64(w) * or_f16_to_f64(Xh[n * K + k]);
    }
    return acc;
}

/*
 * The same whole paths with the rows of Y split into contiguous ranges, one
 * per thread (for timing the oracle on every core of a host). Each thread
 * runs the definitions above on its own rows only: decode of those rows of W
 * (their tiles are a contiguous part of the stream; the stream's offsets are
 * absolute, so no rebasing is needed), the unpacked X, the exact product.
 * The result does not depend on the thread count.
 */
typedef struct {
    int dtype;
    const uint64_t *bitmaps;
    const uint32_t *offsets;
    const void *payload;
    int64_t M, K, N, m0, m1;
    const int8_t *Xd;        /* int4: unpacked X [N][K] */
    const uint16_t *Xh;      /* fp16: X [N][K] */
    int32_t *Y32;            /* int4 result [N][M] */
    double *Yf;              /* fp16 result [N][M] */
    int rc;
} or_rows_job;

static void *or_rows_worker(void *arg) {
    or_rows_job *j = (or_rows_job *)arg;
    int64_t T = or_tiles_per_row(j->K);
    int64_t rows = j->m1 - j->m0;
    j->rc = OR_OK;
    if (rows <= 0) return NULL;
    /* the job's rows as a stream of their own: same words and offsets, the
     * payload pointer unchanged (offsets index it absolutely) */
    const uint64_t *bm = j->bitmaps + j->m0 * T;
    const uint32_t *off = j->offsets + j->m0 * T;
    if (j->dtype == 0) {
        int8_t *Wd = (int8_t *)malloc((size_t)(rows * j->K > 0 ? rows * j->K : 1));
        int64_t *Y64 = (int64_t *)malloc((size_t)(rows * j->N > 0 ? rows * j->N : 1) * sizeof(int64_t));
        if (!Wd || !Y64) { free(Wd); free(Y64); j->rc = OR_E_ARG; return NULL; }
        or_decode(0, bm, off, j->payload, rows, j->K, Wd);
        or_matmul_i64(Wd, rows, j->K, j->Xd, j->N, Y64);    /* Y64[n][r] for the job's rows */
        for (int64_t n = 0; n < j->N; ++n)
            for (int64_t r = 0; r < rows; ++r) {
                int64_t v = Y64[n * rows + r];
                if (v > INT32_MAX || v < INT32_MIN) j->rc = OR_E_OVERFLOW;
                j->Y32[n * j->M + j->m0 + r] = (int32_t)v;
            }
        free(Wd); free(Y64);
    } else {
        uint16_t *Wd = (uint16_t *)malloc((size_t)(rows * j->K > 0 ? rows * j->K : 1) * sizeof(uint16_t));
        double *Yr = (double *)malloc((size_t)(rows * j->N > 0 ? rows * j->N : 1) * sizeof(double));
        if (!Wd || !Yr) { free(Wd); free(Yr); j->rc = OR_E_ARG; return NULL; }
        or_decode(1, bm, off, j->payload, rows, j->K, Wd);
        or_matmul_f64(Wd, rows, j->K, j->Xh, j->N, Yr);
        for (int64_t n = 0; n < j->N; ++n)
            for (int64_t r = 0; r < rows; ++r) j->Yf[n * j->M + j->m0 + r] = Yr[n * rows + r];
        free(Wd); free(Yr);
    }
    return NULL;
}

static int or_spmm_threads(int dtype, const uint64_t *bitmaps, const uint32_t *offsets, const void *payload,
                           int64_t M, int64_t K, const void *X, int64_t N, void *Y, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 1024) nthreads = 1024;
    int8_t *Xd = NULL;
    if (dtype == 0) {
        Xd = (int8_t *)malloc((size_t)(N * K > 0 ? N * K : 1));
        if (!Xd) return OR_E_ARG;
        or_unpack_x4((const uint8_t *)X, N, K, Xd);
    }
    or_rows_job *jobs = (or_rows_job *)calloc((size_t)nthreads, sizeof(or_rows_job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int *started = (int *)calloc((size_t)nthreads, sizeof(int));
    if (!jobs || !th || !started) { free(Xd); free(jobs); free(th); free(started); return OR_E_ARG; }
    for (int i = 0; i < nthreads; ++i) {
        or_rows_job *j = &jobs[i];
        j->dtype = dtype; j->bitmaps = bitmaps; j->offsets = offsets; j->payload = payload;
        j->M = M; j->K = K; j->N = N;
        j->m0 = M * i / nthreads; j->m1 = M * (i + 1) / nthreads;
        j->Xd = Xd; j->Xh = (const uint16_t *)X;
        j->Y32 = (int32_t *)Y; j->Yf = (double *)Y;
        started[i] = pthread_create(&th[i], NULL, or_rows_worker, j) == 0;
        if (!started[i]) or_rows_worker(j);
    }
    int rc = OR_OK;
    for (int i = 0; i < nthreads; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        if (jobs[i].rc != OR_OK) rc = jobs[i].rc;
    }
    free(Xd); free(jobs); free(th); free(started);
    return rc;
}

int or_spmm_w4a4_mt(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                    int64_t M, int64_t K, const uint8_t *Xp, int64_t N, int32_t *Y, int nthreads) {
    return or_spmm_threads(0, bitmaps, offsets, payload, M, K, Xp, N, Y, nthreads);
}

int or_spmm_f16_mt(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                   int64_t M, int64_t K, const uint16_t *Xh, int64_t N, double *Y, int nthreads) {
    return or_spmm_threads(1, bitmaps, offsets, payload, M, K, Xh, N, Y, nthreads);
}
