// spmm.hip -- SpMM entry points of the bitmap-tiled sparse x dense matmul
// for gfx950 (CDNA4): argument checks, kernel selection, launches.
//
// Y = W_sparse * X (SPDP, Sec. 2.2; UnionSparse, Sec. VI) with W in the BT64
// stream (UnionSparse Sec. V-A, one area per 1 x 64 tile) and X a skinny
// K x N activation matrix stored as [N][K]. The kernels live in the
// kernels_*.hip files included below so that one translation unit holds the
// whole device code of the library.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "bitmap_spmm.h"
#include "device_common.h"
#include "kernels_rowwave.hip"
#include "kernels_bt64.hip"
#include "kernels_bt64_f16.hip"

namespace {

struct Shape {
    int64_t M, K, N, T, G;
};

// Host-side validation shared by both dtypes; runs before any HIP call.
int check_args(const void *bitmaps, const void *offsets, const void *payload, int64_t payload_bytes,
               int64_t M, int64_t K, const void *X, int64_t N, const void *Y, int algo, Shape *s) {
    if (M < 0 || K < 0 || N < 0 || payload_bytes < 0) return BSP_E_ARG;
    if (N > BSP_MAX_N) return BSP_E_ARG;
    if (algo < BSP_ALGO_AUTO || algo > BSP_ALGO_MFMA) return BSP_E_ARG;
    if (K >= BSP_MAX_K) return BSP_E_OVERFLOW;
    if (M > INT32_MAX) return BSP_E_OVERFLOW;
    const int64_t T = (K + 63) / 64;
    if (M * T >= INT32_MAX) return BSP_E_OVERFLOW;
    if (payload_bytes % BSP_PAYLOAD_ALIGN != 0) return BSP_E_ARG;
    if (payload_bytes > UINT32_MAX) return BSP_E_OVERFLOW;   // buffer-resource range is 32-bit
    s->M = M; s->K = K; s->N = N; s->T = T; s->G = M * T;
    if (M == 0 || N == 0) return BSP_OK;                     // nothing to compute or write
    if (Y == nullptr || offsets == nullptr) return BSP_E_ARG;
    if (T > 0 && (bitmaps == nullptr || X == nullptr)) return BSP_E_ARG;
    if (payload == nullptr && payload_bytes != 0) return BSP_E_ARG;
    return BSP_OK;
}

int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BSP_OK : BSP_E_HIP;
}

// Whether a kernel family can run a problem (layout constraints of the fast paths).
bool algo_supported(int algo, int dtype, const Shape &s) {
    switch (algo) {
        case BSP_ALGO_ROWWAVE: return true;
        case BSP_ALGO_MFMA: return dtype == BSP_INT4 ? bt64_supported(s.K, s.N) : bf_supported(s.K, s.N);
        default: return false;
    }
}

int select_algo(int dtype, const Shape &s, int64_t nnz) {
    (void)nnz;
    if (algo_supported(BSP_ALGO_MFMA, dtype, s)) return BSP_ALGO_MFMA;
    return BSP_ALGO_ROWWAVE;
}

}  // namespace

extern "C" int bsp_select(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz) {
    if (dtype != BSP_INT4 && dtype != BSP_FP16) return -1;
    if (M < 0 || K < 0 || N < 0 || N > BSP_MAX_N) return -1;
    Shape s{M, K, N, (K + 63) / 64, M * ((K + 63) / 64)};
    return select_algo(dtype, s, nnz);
}

extern "C" int bsp_describe_selection(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz,
                                      char *buf, size_t n) {
    int a = bsp_select(dtype, M, K, N, nnz);
    if (a < 0 || buf == nullptr || n == 0) return BSP_E_ARG;
    const char *name = a == BSP_ALGO_ROWWAVE ? "rowwave" : "mfma";
    const char *ty = dtype == BSP_INT4 ? "int4" : "fp16";
    // payload bytes the encoder writes for nnz nonzeros (all of W when unknown)
    const int64_t nz = nnz >= 0 ? nnz : M * K;
    const int64_t pbytes = dtype == BSP_INT4 ? (nz + 1) / 2 : 2 * nz;
    char launch[160] = "";
    if (a == BSP_ALGO_MFMA && M > 0 && N > 0) {
        if (dtype == BSP_INT4) {
            BtPlan p;
            if (bt64_plan(M, K, N, pbytes, &p)) {
                if (p.streaming)
                    snprintf(launch, sizeof launch, " kernel=k_bt64s_w4a4 grid=%u block=%d lds=%zu stage_kb=%d stagger=%d",
                             p.grid, 64 * p.nwaves, p.lds, p.area_kb, p.stagger);
                else
                    snprintf(launch, sizeof launch, " kernel=k_bt64_w4a4 grid=%u block=%d lds=%zu tiles_per_lane=%d one_pass=%d",
                             p.grid, 64 * p.nwaves, p.lds, p.tpl, p.one_pass);
            }
        } else {
            Bf8Plan p8;
            BfPlan p;
            if (bf8_plan(M, K, N, pbytes, &p8))
                snprintf(launch, sizeof launch, " kernel=k_bt8_f16 grid=%u block=%d lds=%zu stage_kb=%u step_slots=%d",
                         p8.grid, 64 * p8.nwaves, p8.lds, p8.area_kb, p8.nstep);
            else if (bf_plan(M, K, N, pbytes, &p))
                snprintf(launch, sizeof launch, " kernel=k_bt64_f16 grid=%u block=%d lds=%zu", p.grid, 64 * p.nwaves,
                         p.lds);
        }
    }
    if (launch[0] == 0 && M > 0 && N > 0)
        snprintf(launch, sizeof launch, " kernel=k_rowwave_%s", dtype == BSP_INT4 ? "w4a4" : "f16");
    snprintf(buf, n, "dtype=%s M=%lld K=%lld N=%lld nnz=%lld -> %s%s", ty, (long long)M, (long long)K, (long long)N,
             (long long)nnz, name, launch);
    return BSP_OK;
}

extern "C" int spmm_bitmap_w4a4_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                     int64_t payload_bytes, int64_t M, int64_t K,
                                     const uint8_t *X, int64_t N, int32_t *Y, int algo, hipStream_t stream) {
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, algo, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    // The MFMA kernels read X in whole dwords from its start (the last one
    // may reach up to 3 bytes past N * ceil(K/2), inside the same page only
    // when X starts on a 4-byte boundary): an X off that boundary takes the
    // plain kernel.
    const bool x_aligned = ((uintptr_t)X & 3u) == 0;
    if (algo == BSP_ALGO_AUTO) {
        algo = select_algo(BSP_INT4, s, -1);
        if (algo == BSP_ALGO_MFMA && !x_aligned) algo = BSP_ALGO_ROWWAVE;
    }
    if (!algo_supported(algo, BSP_INT4, s) || (algo == BSP_ALGO_MFMA && !x_aligned))
        return BSP_E_UNSUPPORTED;   // a forced kernel never falls back
    switch (algo) {
        case BSP_ALGO_MFMA: {
            BtPlan plan;
            if (!bt64_plan(M, K, N, payload_bytes, &plan)) return BSP_E_UNSUPPORTED;
            launch_bt64_w4a4(plan, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N,
                             Y, stream);
            break;
        }
        default:
        case BSP_ALGO_ROWWAVE:
            launch_rowwave_w4a4(bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K,
                                X, (int)N, Y, stream);
            break;
    }
    return launch_status();
}

extern "C" int spmm_bitmap_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                int64_t payload_bytes, int64_t M, int64_t K,
                                const uint8_t *X, int64_t N, int32_t *Y, hipStream_t stream) {
    return spmm_bitmap_w4a4_algo(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, BSP_ALGO_AUTO, stream);
}

extern "C" int spmm_bitmap_f16_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                                    int64_t payload_bytes, int64_t M, int64_t K,
                                    const uint16_t *X, int64_t N, uint16_t *Y, int algo, hipStream_t stream) {
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, algo, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    if (algo == BSP_ALGO_AUTO) algo = select_algo(BSP_FP16, s, -1);
    if (!algo_supported(algo, BSP_FP16, s)) return BSP_E_UNSUPPORTED;   // a forced kernel never falls back
    switch (algo) {
        case BSP_ALGO_MFMA: {
            Bf8Plan plan8;
            if (bf8_plan(M, K, N, payload_bytes, &plan8)) {
                launch_bt8_f16(plan8, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, Y,
                               stream);
                break;
            }
            BfPlan plan;
            if (!bf_plan(M, K, N, payload_bytes, &plan)) return BSP_E_UNSUPPORTED;
            launch_bt64_f16(plan, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N,
                            Y, stream);
            break;
        }
        default:
        case BSP_ALGO_ROWWAVE:
            launch_rowwave_f16(bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K,
                               X, (int)N, Y, stream);
            break;
    }
    return launch_status();
}

extern "C" int spmm_bitmap_f16(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                               int64_t payload_bytes, int64_t M, int64_t K,
                               const uint16_t *X, int64_t N, uint16_t *Y, hipStream_t stream) {
    return spmm_bitmap_f16_algo(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, BSP_ALGO_AUTO, stream);
}
