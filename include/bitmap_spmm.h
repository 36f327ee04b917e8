/*
 * bitmap_spmm.h -- C ABI of the bitmap-tiled sparse x dense matmul for AMD
 * Instinct MI355X (gfx950).
 *
 * Computes Y = W_sparse * X, the problem statement of SPDP ("Unified
 * Static-Dynamic Pruning for Efficient LLM Inference", Sec. 2.2) and of the
 * UnionSparse SpMM kernel ("UnionSparse: An Index-Efficient Sparsity
 * Framework for Low-Bit Sparse LLM Inference on Edge", IEEE TCAD, Sec. VI),
 * for the decode-phase shapes those pages study: W is M x K with 30-70 %
 * unstructured sparsity, X is a skinny K x N activation matrix, N = 1..32.
 *
 * ---------------------------------------------------------------------------
 * Encoded format ("BT64"): UnionSparse Sec. V-A, "IE-BME Representation",
 * with one area per tile (R_A = C_A = 1, Q = 1) on 1 x 64 row tiles.
 *   T = ceil(K/64) tiles per row; G = M*T tiles; tile g = m*T + t covers
 *   columns 64t .. 64t+63 of row m (row-major tile order).
 *   bitmaps[g]   uint64. Bit j is set iff W[m][64t+j] != 0; bit 0 is the
 *                first column (the LSB-first packing of the Fig. 7 example).
 *                Bits of columns >= K are zero.
 *   offsets[g]   uint32, the number of nonzeros in tiles 0..g-1 ("Union Value
 *                Offsets" with Q = 1); offsets[G] = nnz. G+1 entries.
 *   payload      the nonzeros in tile order and, inside a tile, in column
 *                order: value (m, 64t+j) is element offsets[g] + rank, rank =
 *                popcount(bitmaps[g] & ((1<<j)-1)) ("Compressed Values").
 *                int4: element e is byte e>>1, low nibble when e is even, a
 *                4-bit two's-complement code; ceil(nnz/2) bytes, an odd count
 *                leaves the final high nibble zero.
 *                fp16: element e is uint16 e (IEEE binary16 bits); 2*nnz bytes.
 * Activations: X is K x N stored column by column, i.e. an [N][K] array.
 *   int4: packed along K, two per byte, low nibble = even k, row stride
 *   ceil(K/2) bytes. fp16: row stride K elements.
 * Output: Y is M x N stored column by column, i.e. [N][M]; int32 for the int4
 *   path, fp16 for the fp16 path. Y is fully overwritten, never accumulated.
 * ---------------------------------------------------------------------------
 *
 * Conventions
 *   - Every entry point returns a bsp_status. No C++ exception crosses the ABI.
 *   - Arguments are checked on the host before any HIP call, so a bad call
 *     returns an error code without touching the GPU.
 *   - SpMM calls are asynchronous on `stream` (NULL = the null stream); a fault
 *     inside a kernel surfaces at the caller's next synchronisation. The
 *     content of the encoded stream is not validated on the device (that
 *     would cost a full extra pass over HBM): a corrupt stream gives a wrong
 *     Y, never an out-of-bounds access, because every payload read is bounded
 *     by `payload_bytes` in hardware (buffer-resource loads).
 *   - The calls hold no state between calls, allocate no memory and are
 *     reentrant; concurrent calls on different streams are allowed.
 */
#ifndef BITMAP_SPMM_H
#define BITMAP_SPMM_H

#include <stdint.h>
#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsp_status {
    BSP_OK = 0,
    BSP_E_ARG = 1,       /* null pointer, negative size, N > 32, ldw < K, unknown dtype/algo */
    BSP_E_RANGE = 2,     /* a weight outside its type's range: int4 [-8, 7], int2 [-2, 1] */
    BSP_E_CAPACITY = 3,  /* payload buffer smaller than the encoded payload */
    BSP_E_OVERFLOW = 4,  /* nnz >= 2^32, K >= 2^25 (int32 sums could overflow), or an index beyond 2^31 */
    BSP_E_HIP = 5,       /* a HIP launch error (hipGetLastError after the launch) */
    BSP_E_UNSUPPORTED = 6 /* a kernel forced through an *_algo entry point cannot run this shape */
} bsp_status;

typedef enum bsp_dtype { BSP_INT4 = 0, BSP_FP16 = 1, BSP_INT2 = 2 } bsp_dtype;

/* Kernel choice for the *_algo entry points. BSP_ALGO_AUTO applies the
 * library's shape-aware selection (by N, density, M, K). A forced choice
 * that cannot run the shape returns BSP_E_UNSUPPORTED and launches nothing;
 * it never falls back to another kernel. */
typedef enum bsp_algo {
    BSP_ALGO_AUTO = 0,
    BSP_ALGO_ROWWAVE = 1,   /* one wavefront per output row; plain per-nonzero decode (any shape) */
    BSP_ALGO_MFMA = 2,      /* lane-per-tile decode from LDS-staged 16-row blocks over all of K + int8 / fp16
                               MFMA (int4: K <= 16384; fp16: K <= 4096, K % 8 == 0) */
    BSP_ALGO_SPLITK = 3     /* the same decode and MFMA over K ranges of block sets (UnionSparse Sec. VI-C,
                               Alg. 2: partial tiles, then a reduction): any K (fp16: K % 8 == 0); with a
                               workspace (the *_ws entry points) a block set's K ranges run on several
                               workgroups and meet in it */
} bsp_algo;

/* The device payload allocation handed to the SpMM calls is a whole number
 * of 16-byte units (zero-filled past the encoded payload): kernels read it in
 * whole dwords, and the hardware range check is applied to whole dwords. */
#define BSP_PAYLOAD_ALIGN 16

/* Largest N the SpMM entry points accept. */
#define BSP_MAX_N 32
/* K bound that keeps every int4 x int4 sum inside int32: |Y| <= 64*K < 2^31. */
#define BSP_MAX_K ((int64_t)1 << 25)

/*
 * encode_bitmap_tiles -- host-side encoder (UnionSparse Sec. V-A, Q = 1 on
 * 1 x 64 tiles; the encoded form is produced offline and cached, Sec. V-B).
 *
 *   dtype    BSP_INT4: W is const int8_t*, values in [-8, 7];
 *            BSP_INT2: W is const int8_t*, values in [-2, 1] (the W2A4 weights
 *            of UnionSparse Sec. VII, Fig. 11): payload element e is the 2-bit
 *            two's-complement code in byte e>>2 at bits 2*(e&3), lowest first;
 *            BSP_FP16: W is const uint16_t* holding IEEE binary16 bits
 *            (+0 and -0 are zero; every other pattern, NaN included, is stored).
 *   W        HOST memory, row-major M x K with leading dimension ldw >= K.
 *   bitmaps  HOST, caller-allocated, M*T entries (T = ceil(K/64)), or NULL.
 *   offsets  HOST, caller-allocated, M*T+1 entries, or NULL.
 *   payload  HOST, caller-allocated, payload_capacity_bytes bytes, or NULL for
 *            a size query (then bitmaps/offsets may also be NULL).
 *   nnz_out, payload_bytes_out  written on BSP_OK and on BSP_E_CAPACITY
 *            (either may be NULL). payload_bytes = ceil(nnz/2) (int4),
 *            ceil(nnz/4) (int2) or 2*nnz (fp16).
 * Returns BSP_E_ARG, BSP_E_RANGE (nothing written), BSP_E_OVERFLOW
 * (nnz >= 2^32), BSP_E_CAPACITY (counts written, arrays untouched) or BSP_OK.
 * Multi-threaded over rows; the output does not depend on the thread count.
 */
int encode_bitmap_tiles(int dtype, const void *W, int64_t M, int64_t K, int64_t ldw,
                        uint64_t *bitmaps, uint32_t *offsets,
                        void *payload, int64_t payload_capacity_bytes,
                        int64_t *nnz_out, int64_t *payload_bytes_out);

/*
 * pack_int4_activations -- host helper that writes int4 activations in the
 * layout the SpMM reads: X (values in [-8, 7], HOST [N][K] int8, row stride
 * ldx >= K) -> Xp (HOST, N * ceil(K/2) bytes). Returns BSP_E_RANGE for a
 * value outside [-8, 7] (Xp then undefined).
 */
int pack_int4_activations(const int8_t *X, int64_t N, int64_t K, int64_t ldx, uint8_t *Xp);

/*
 * spmm_bitmap_w4a4 -- Y = W * X with int4 W (BT64 stream) and int4 X, exact
 * int32 result (UnionSparse Sec. VI; W4A4 decode shapes of Sec. VII-A).
 *
 *   bitmaps, offsets, payload   DEVICE, the encoded W (M*T, M*T+1 entries and
 *                               payload_bytes bytes); payload may be NULL only
 *                               if payload_bytes == 0.
 *   payload_bytes               size of the payload allocation: a multiple of
 *                               BSP_PAYLOAD_ALIGN, >= ceil(nnz/2), bytes past the
 *                               encoded payload zero. No byte at or past it is read.
 *   M, K                        0 <= M < 2^31, 0 <= K < 2^25, M*ceil(K/64) < 2^31.
 *   X                           DEVICE, [N][ceil(K/2)] packed int4. The MFMA and split-K
 *                               kernels need X on a 4-byte boundary (any allocation is;
 *                               fp16: 16 bytes); an X off it runs the plain kernel
 *                               (BSP_ALGO_AUTO) or is refused with BSP_E_UNSUPPORTED.
 *   N                           0..32. N == 0 or M == 0: nothing is launched.
 *   Y                           DEVICE, [N][M] int32, fully overwritten (K == 0 gives zeros).
 *   stream                      HIP stream (NULL = null stream).
 * Exact: int32 sums are associative and cannot overflow under the K bound,
 * so every kernel gives the same bits.
 */
int spmm_bitmap_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                     int64_t payload_bytes, int64_t M, int64_t K,
                     const uint8_t *X, int64_t N, int32_t *Y, hipStream_t stream);

/* As spmm_bitmap_w4a4 with an explicit kernel choice (bsp_algo). */
int spmm_bitmap_w4a4_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                          int64_t payload_bytes, int64_t M, int64_t K,
                          const uint8_t *X, int64_t N, int32_t *Y, int algo, hipStream_t stream);

/*
 * spmm_bitmap_f16 -- fp16 variant (SPDP Sec. 4: FP16 values in a bitmap
 * format, decoded with a masked-popcount rank): payload is uint16[nnz]
 * (payload_bytes >= 2*nnz, a multiple of BSP_PAYLOAD_ALIGN), X is fp16 [N][K],
 * Y is fp16 [N][M]. Products and
 * sums in fp32 (any order), one round-to-nearest-even to fp16 at the end.
 * Other arguments as spmm_bitmap_w4a4.
 */
int spmm_bitmap_f16(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                    int64_t payload_bytes, int64_t M, int64_t K,
                    const uint16_t *X, int64_t N, uint16_t *Y, hipStream_t stream);

int spmm_bitmap_f16_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                         int64_t payload_bytes, int64_t M, int64_t K,
                         const uint16_t *X, int64_t N, uint16_t *Y, int algo, hipStream_t stream);

/*
 * Split-K with a workspace (UnionSparse Sec. VI-C, Alg. 2: each workgroup
 * stores its partial tile, a reduction adds them; the N:M co-design page,
 * Sec. 4.3, bounds the split count). The library allocates nothing; callers
 * that want the split plans pass a workspace:
 *
 *   bsp_workspace_bytes -- bytes of workspace the *_ws entry points want for
 *     a problem (their automatic plan and the forced BSP_ALGO_SPLITK plan),
 *     0 when no plan of the shape uses one. nnz may be -1 when unknown.
 *     Returns BSP_E_ARG / BSP_E_OVERFLOW for invalid shapes. Host only.
 *
 *   spmm_bitmap_w4a4_ws / spmm_bitmap_f16_ws -- as the *_algo entry points
 *     with a workspace: DEVICE memory, 256-byte aligned, workspace_bytes long,
 *     owned by the caller, ZERO-FILLED before its first use (its first 64 KiB
 *     hold arrival counters; every call leaves them at zero again, so one
 *     workspace serves calls of any shapes in turn). workspace may be NULL
 *     with workspace_bytes 0 (then no plan needs one). A plan that needs more
 *     than workspace_bytes returns BSP_E_CAPACITY and launches nothing; a
 *     workspace off a 256-byte boundary returns BSP_E_ARG. Calls that share a
 *     workspace must be ordered (one stream, or events): concurrent calls on
 *     one workspace race. fp16 results do not depend on timing (partials are
 *     added in a fixed order).
 */
int bsp_workspace_bytes(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, int64_t *bytes);

int spmm_bitmap_w4a4_ws(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                        int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N, int32_t *Y,
                        void *workspace, int64_t workspace_bytes, int algo, hipStream_t stream);

int spmm_bitmap_f16_ws(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                       int64_t payload_bytes, int64_t M, int64_t K, const uint16_t *X, int64_t N, uint16_t *Y,
                       void *workspace, int64_t workspace_bytes, int algo, hipStream_t stream);

/*
 * spmm_bitmap_f16_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): spmm_bitmap_f16_ws with the library's own scratch as the
 * workspace instead of a caller's. The scratch is a static device array of
 * bsp_noalloc_scratch_bytes() bytes (8 MiB), one per GPU, held until the
 * process ends; its device address is looked up on a device's first call
 * (which also clears it with a fill kernel on `stream`). No call allocates.
 * A plan that needs more scratch returns BSP_E_CAPACITY (a 4096-row fp16
 * problem needs at most 1 MiB; the need grows with M and N). Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams without ordering) race, and must not be made. Other arguments,
 * results and errors as spmm_bitmap_f16_ws.
 */
int spmm_bitmap_f16_noalloc(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                            int64_t payload_bytes, int64_t M, int64_t K, const uint16_t *X, int64_t N,
                            uint16_t *Y, int algo, hipStream_t stream);

/* Size in bytes of the per-GPU scratch of spmm_bitmap_f16_noalloc. */
int64_t bsp_noalloc_scratch_bytes(void);

/*
 * bsp_select -- the kernel BSP_ALGO_AUTO picks for a problem (shape-aware
 * selection; UnionSparse Sec. I names it, without a rule). nnz may be -1 when
 * unknown. Returns a bsp_algo value, or -1 for invalid arguments. Host only.
 */
int bsp_select(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz);

/* Human-readable description of bsp_select's choice and launch shape (the
 * plain and *_algo entry points, no workspace), written NUL-terminated into
 * buf (at most n bytes). Returns bsp_status. Host only. */
int bsp_describe_selection(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, char *buf, size_t n);

/* The same for the automatic plan of the *_ws entry points given a
 * workspace of bsp_workspace_bytes. */
int bsp_describe_selection_ws(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, char *buf, size_t n);

/* The plan an explicit kernel choice takes: `algo` (a bsp_algo) through the
 * *_algo entry points (with_workspace 0) or the *_ws ones given a workspace
 * of bsp_workspace_bytes (with_workspace 1), described as above. Returns
 * BSP_E_UNSUPPORTED (and a description saying so) when that choice cannot
 * run the shape, BSP_E_ARG for an unknown dtype or algo. Host only. */
int bsp_describe_plan(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, int algo, int with_workspace,
                      char *buf, size_t n);

/*
 * spmm_bitmap_w2a4 -- Y = W * X with W's values 2-bit (encoded with dtype
 * BSP_INT2: the W2A4 setting of UnionSparse Sec. VII, Fig. 11) and X packed
 * int4 as for spmm_bitmap_w4a4; Y int32 [N][M], exact. payload_bytes >=
 * ceil(nnz/4), a multiple of BSP_PAYLOAD_ALIGN. The automatic choice runs the
 * MFMA block kernels (streaming up to K = 4096, the ring kernel up to 16384;
 * X on a 4-byte boundary) and the plain kernel elsewhere; _algo forces
 * BSP_ALGO_MFMA (BSP_E_UNSUPPORTED outside it) or BSP_ALGO_ROWWAVE;
 * BSP_ALGO_SPLITK returns BSP_E_UNSUPPORTED. bsp_describe_selection and
 * bsp_describe_plan with dtype BSP_INT2 describe these plans.
 */
int spmm_bitmap_w2a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                     int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                     int32_t *Y, hipStream_t stream);
int spmm_bitmap_w2a4_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                          int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                          int32_t *Y, int algo, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Dequant epilogue and grouped launch (the Quant -> SpMM -> Dequant pipeline
 * of UnionSparse Fig. 2, with the Dequant step fused into the SpMM's final
 * write, and several matrices in one launch).
 * With the epilogue, output element (n, m) is
 *     Yh[n*M + m] = fp16( fp32( fp32(y) * scale_w[m] ) * scale_x[n] )
 * y being the int32 sum of spmm_bitmap_w4a4: the sum converted to fp32
 * (round to nearest even), multiplied by the output channel's scale, then by
 * the token's scale, each product rounded to nearest even in fp32, and one
 * round to nearest even to fp16 (overflow gives +-inf). Scales are fp32, in
 * the normal range (no subnormal products).
 * --------------------------------------------------------------------------- */

/*
 * spmm_bitmap_w4a4_dq -- spmm_bitmap_w4a4 with the dequant epilogue.
 *   scale_w    DEVICE float[M], one scale per output row (channel).
 *   scale_x    DEVICE float[N], one scale per activation column (token).
 *   Yh         DEVICE uint16 [N][M] (fp16 bits), fully overwritten.
 * Runs the int4 MFMA kernels (K <= 16384, X on a 4-byte boundary); other
 * shapes return BSP_E_UNSUPPORTED. K == 0 gives fp16(0 * scale_w * scale_x)
 * (signed zeros). Other arguments as spmm_bitmap_w4a4.
 */
int spmm_bitmap_w4a4_dq(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                        int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                        const float *scale_w, const float *scale_x, uint16_t *Yh, hipStream_t stream);

/* Most matrices in one grouped launch. */
#define BSP_GROUP_MAX 8

/* One matrix of a grouped launch: its BT64 stream, its X, and exactly one of
 * Y (int32 [N][M]) or Yh (fp16 [N][M] through the dequant epilogue, with
 * scale_w[M] and scale_x[N]). All pointers DEVICE; M, N, payload_bytes as for
 * spmm_bitmap_w4a4. An item with M == 0 or N == 0 is skipped. */
typedef struct bsp_w4a4_item {
    const uint64_t *bitmaps;
    const uint32_t *offsets;
    const uint8_t *payload;
    int64_t payload_bytes;
    int64_t M;
    const uint8_t *X;
    int64_t N;
    int32_t *Y;
    uint16_t *Yh;
    const float *scale_w;
    const float *scale_x;
} bsp_w4a4_item;

/*
 * spmm_bitmap_w4a4_grouped -- Y_i = W_i * X_i for `count` (1..BSP_GROUP_MAX)
 * matrices sharing one K (e.g. the Q, K and V projections of a layer, or an
 * FFN's gate and up projections) in ONE kernel launch on `stream`; the
 * workgroups are shared out over the items in proportion to their rows.
 *   items      HOST array of `count` descriptors (read during the call only).
 * Results equal spmm_bitmap_w4a4 / spmm_bitmap_w4a4_dq per item, bit for bit.
 * The items must all run the streaming int4 kernel (1 <= K <= 4096, X on a
 * 4-byte boundary), else BSP_E_UNSUPPORTED and nothing is launched. Errors
 * in any item are reported before anything is launched.
 */
int spmm_bitmap_w4a4_grouped(const bsp_w4a4_item *items, int count, int64_t K, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Union-mask format ("IE-BME"): UnionSparse Sec. V-A, Fig. 7, with 16 x 64
 * local tiles (LTs) and bitmap-aware row reordering (Sec. V-B, Eq. 3-5,
 * Algorithm 1).
 *   bands = ceil(M/16), T = ceil(K/64), nlt = bands*T LTs in row-major order
 *   (LT t = band*T + column covers rows 16*band .. +15, columns 64*column ..
 *   +63; past M or K the tile is padded with zeros).
 *   An LT is cut into ra x ca areas of (16/ra) x (64/ca); area q = a*ca + c
 *   holds tile rows a*16/ra .. and columns c*64/ca ... Logical position (i, j)
 *   of the (16/ra) x (64/ca) union mask is set iff any area has a nonzero at
 *   (i, j) (after the LT's row permutation).
 *   ubitmaps[t*W .. t*W+W-1]  uint64, W = 16/(ra*ca) words: the mask scanned
 *                row-major, position f in bit f%64 of word f/64 (leftmost
 *                position of a row in the lowest bit, as in Fig. 7).
 *   offsets[t]   uint32, number of values before LT t ("Union Value Offsets":
 *                the sum of Q*P over earlier LTs, Q = ra*ca, P = set mask
 *                bits); offsets[nlt] = nvals. nlt+1 entries.
 *   rowpos[t]    uint64, nibble r = position of tile row r in the LT's
 *                reordered row order (identity without reordering). The
 *                reordered tile lists, area row by area row, row p of every
 *                row group found by the reordering.
 *   payload      int4 values ("Compressed Values"): for each set position of
 *                rank rho (set positions before it, row-major), area q's value
 *                (zero or not) is element offsets[t] + q*P + rho. Element e is
 *                byte e>>1, low nibble when e is even. ceil(nvals/2) bytes.
 * Row reordering, per LT: rows are grouped into 16/ra groups of ra rows so
 * that the number of set mask positions is minimal (subset DP over row sets,
 * each step taking a group with the smallest remaining row); among equal
 * costs the first group in ascending lexicographic order is kept.
 * --------------------------------------------------------------------------- */
#define BSP_LT_ROWS 16
#define BSP_LT_COLS 64

/* Number of LTs of an M x K matrix (ceil(M/16)*ceil(K/64)); -1 for negative sizes. */
int64_t union_tile_count(int64_t M, int64_t K);

/* 64-bit mask words per LT for an ra x ca partition: 16/(ra*ca). 0 when the
 * partition is not supported (ra, ca powers of two with ra*ca <= 16). */
int union_mask_words(int ra, int ca);

/*
 * encode_union_tiles -- host-side encoder of the union-mask format.
 *   W          HOST int8 [M][ldw], values in [-8, 7] (BSP_E_RANGE otherwise).
 *   ra, ca     area partition (union_mask_words(ra, ca) > 0, else BSP_E_ARG).
 *   reorder    nonzero: bitmap-aware row reordering of every LT; 0: identity.
 *   ubitmaps, offsets, rowpos   HOST, caller-allocated: nlt*W, nlt+1 and nlt
 *              entries; all three NULL for a size query.
 *   payload    HOST, payload_capacity_bytes >= ceil(nvals/2), or NULL (size
 *              query, or words/offsets/rowpos only).
 *   nvals_out, payload_bytes_out  written on BSP_OK, BSP_E_CAPACITY and
 *              BSP_E_OVERFLOW (either may be NULL).
 * Returns BSP_E_OVERFLOW when nvals >= 2^32. Deterministic for a given input.
 */
int encode_union_tiles(const int8_t *W, int64_t M, int64_t K, int64_t ldw, int ra, int ca, int reorder,
                       uint64_t *ubitmaps, uint32_t *offsets, uint64_t *rowpos,
                       uint8_t *payload, int64_t payload_capacity_bytes,
                       int64_t *nvals_out, int64_t *payload_bytes_out);

/* K bound of the union-mask SpMM. */
#define BSP_UNION_MAX_K 32768

/*
 * spmm_union_w4a4 -- Y = W * X with W in the union-mask format (int4 values,
 * int32 Y), asynchronous on `stream`. All pointers are DEVICE memory.
 *   ubitmaps, offsets, rowpos, payload   as encode_union_tiles wrote them;
 *              payload_bytes is the payload allocation (a multiple of
 *              BSP_PAYLOAD_ALIGN, zero past the encoded bytes).
 *   ra, ca     the encoding's partition. The kernel runs ra = ca = 2 (the
 *              pages' 2 x 2 areas); another valid partition returns
 *              BSP_E_UNSUPPORTED, an invalid one BSP_E_ARG.
 *   M, K       0 <= M < 2^31, 0 <= K <= BSP_UNION_MAX_K (larger K: BSP_E_UNSUPPORTED).
 *   X          [N][ceil(K/2)] packed int4 as for spmm_bitmap_w4a4, on a 4-byte
 *              boundary (BSP_E_UNSUPPORTED otherwise).
 *   N          0..32; N == 0 or M == 0 launches nothing.
 *   Y          [N][M] int32, fully overwritten (K == 0 gives zeros).
 */
int spmm_union_w4a4(const uint64_t *ubitmaps, const uint32_t *offsets, const uint64_t *rowpos,
                    const uint8_t *payload, int64_t payload_bytes, int ra, int ca, int64_t M, int64_t K,
                    const uint8_t *X, int64_t N, int32_t *Y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Tiled-CBC format and dynamic activation pruning (SPDP, Sec. 4.1 "Tiled-CBC",
 * Fig. 4(a); Sec. 4.2, the decode-phase spMspV kernel).
 *   GTiles of BSP_CBC_TILE_M x BSP_CBC_TILE_K (256 x 64) in row-major order
 *   over the matrix (n_gt = cbc_gtile_count(M, K); zero-padded past M and K).
 *   tile_offsets[g]   uint32, GTile g's first value; n_gt+1 entries, the last NNZ.
 *   colinfo[g*64 + c] uint32, (first value of column c inside the GTile << 16)
 *                     | (nonzeros of column c).
 *   bitmaps[(g*64 + c)*4 + w]  uint64: bit j is row 64w+j of column c.
 *   values            fp16 bits: GTile by GTile, column by column, rows ascending.
 * Storage: 4(n_gt+1) + 4 n_gt 64 + 8 (n_gt 64 4) + 2 NNZ bytes.
 * --------------------------------------------------------------------------- */
#define BSP_CBC_TILE_M 256
#define BSP_CBC_TILE_K 64
/* Largest N of spmspv_cbc_f16 (decode widths). */
#define BSP_CBC_MAX_N 8

/* GTiles of an M x K matrix; -1 for negative sizes. */
int64_t cbc_gtile_count(int64_t M, int64_t K);

/*
 * encode_cbc_f16 -- host-side Tiled-CBC encoder. W: HOST uint16 (fp16 bits)
 * [M][ldw]; +0 and -0 are zero. tile_offsets/colinfo/bitmaps: HOST arrays of
 * n_gt+1, n_gt*64 and n_gt*256 entries, all NULL for a size query; values:
 * HOST, values_capacity elements (>= NNZ), or NULL. nnz_out written on BSP_OK,
 * BSP_E_CAPACITY and BSP_E_OVERFLOW (NNZ >= 2^32).
 */
int encode_cbc_f16(const uint16_t *W, int64_t M, int64_t K, int64_t ldw, uint32_t *tile_offsets,
                   uint32_t *colinfo, uint64_t *bitmaps, uint16_t *values, int64_t values_capacity,
                   int64_t *nnz_out);

/* Workspace bytes spmspv_cbc_f16 uses to split K over workgroups (0: none). */
int spmspv_cbc_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t *bytes);

/*
 * spmspv_cbc_f16 -- Y = W * X' on `stream`, X' = X with every activation of
 * magnitude <= threshold set to zero (dynamic pruning); the columns of W
 * whose activations are all pruned are not read. fp32 products and sums, one
 * round to nearest even to fp16.
 *   tile_offsets, colinfo, bitmaps, values  DEVICE, as encode_cbc_f16 wrote
 *            them; values_bytes: the values allocation, a multiple of
 *            BSP_PAYLOAD_ALIGN, zero past the encoded values.
 *   X        DEVICE fp16 [N][K]; N 0..BSP_CBC_MAX_N.
 *   threshold  fp32, finite, >= 0 (0: the plain product); compared with |x| in fp32.
 *   Y        DEVICE fp16 [N][M], fully overwritten (K == 0 gives zeros).
 *   workspace  DEVICE, NULL (one workgroup per 256-row band) or
 *            spmspv_cbc_workspace_bytes() bytes, 256-byte aligned, zero-filled
 *            before its first use (its first 64 KiB are arrival counters,
 *            left zero by every call); calls that share a workspace must be
 *            ordered on one stream. Too small: BSP_E_CAPACITY.
 */
int spmspv_cbc_f16(const uint32_t *tile_offsets, const uint32_t *colinfo, const uint64_t *bitmaps,
                   const uint16_t *values, int64_t values_bytes, int64_t M, int64_t K, const uint16_t *X,
                   int64_t N, float threshold, uint16_t *Y, void *workspace, int64_t workspace_bytes,
                   hipStream_t stream);

/* Static string for a bsp_status code. */
const char *bsp_status_string(int status);

/* Library version as "major.minor.patch". */
const char *bsp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITMAP_SPMM_H */
