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
#include <mutex>

#include "bitmap_spmm.h"
#include "device_common.h"
#include "kernels_rowwave.hip"
#include "kernels_bt64.hip"
#include "kernels_bt64_f16.hip"
#include "kernels_splitk.hip"
#include "kernels_union.hip"
#include "kernels_cbc.hip"

namespace {

struct Shape {
    int64_t M, K, N, T, G;
};

// Host-side validation shared by both dtypes; runs before any HIP call.
int check_args(const void *bitmaps, const void *offsets, const void *payload, int64_t payload_bytes,
               int64_t M, int64_t K, const void *X, int64_t N, const void *Y, int algo, Shape *s) {
    if (M < 0 || K < 0 || N < 0 || payload_bytes < 0) return BSP_E_ARG;
    if (N > BSP_MAX_N) return BSP_E_ARG;
    if (algo < BSP_ALGO_AUTO || algo > BSP_ALGO_SPLITK) return BSP_E_ARG;
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

// A chosen kernel and its launch shape.
enum PlanKind { PK_ROWWAVE = 0, PK_BT64, PK_BT8F16, PK_BT64F16, PK_BSK };
struct Plan {
    int kind = PK_ROWWAVE;
    int algo = BSP_ALGO_ROWWAVE;
    BtPlan bt;
    Bf8Plan bf8;
    BfPlan bf;
    SkPlan sk;
    int64_t ws_bytes() const { return kind == PK_BSK ? sk.ws_bytes : 0; }
};

// K ranges per block set the automatic plan gives the split-K kernels when
// a workspace is given: 2 for fp16 past K = 4096 (4096 x 11008: 28.1 us
// against 31.0 at N = 8, 26.0 against 27.2 at N = 1); for int4, 2 past
// K = 20480 (T > 320) and 1 up to it (4096 x K at N = 8, 1 against 2
// ranges: K = 20480 22.4 / 24.2 us, 24576 26.1 / 24.1, 28672 29.7 / 30.0,
// 32768 34.7 / 31.9; 4096 x 24576 at N = 32 35.8 / 31.0; 8192 x 24576 at
// N = 8 50.0 / 46.6).
int preferred_splits(int dtype, const Shape &s) {
    if (dtype == BSP_FP16) return s.T > 64 ? 2 : 1;
    return s.T > 320 ? 2 : 1;
}

// The MFMA family: the 16-row block kernels (int4: streaming up to K = 4096,
// ring above, up to K = 16384; fp16: eight-row steps at N <= 8, 16-row
// blocks above, K <= 4096 and K % 8 == 0).
bool plan_mfma(int dtype, const Shape &s, int64_t pbytes, Plan *p) {
    p->algo = BSP_ALGO_MFMA;
    if (dtype == BSP_INT4) {
        if (!bt64_plan(s.M, s.K, s.N, pbytes, &p->bt)) return false;
        p->kind = PK_BT64;
        return true;
    }
    if (bf8_plan(s.M, s.K, s.N, pbytes, &p->bf8)) {
        p->kind = PK_BT8F16;
        return true;
    }
    if (!bf_plan(s.M, s.K, s.N, pbytes, &p->bf)) return false;
    p->kind = PK_BT64F16;
    return true;
}

// The split-K family: any K (fp16: K % 8 == 0), `splits` K ranges per block
// set (fewer if the shape cannot take them; 1 without a workspace).
bool plan_splitk(int dtype, const Shape &s, int64_t pbytes, int splits, Plan *p) {
    p->algo = BSP_ALGO_SPLITK;
    if (dtype == BSP_FP16 && s.K % 8 != 0) return false;
    if (dtype == BSP_INT4 && splits > 1 && sks_plan(s.M, s.K, s.N, pbytes, splits, &p->sk)) {
        p->kind = PK_BSK;
        return true;
    }
    for (; splits >= 1; splits /= 2)
        if (sk_plan(dtype, s.M, s.K, s.N, pbytes, splits, &p->sk)) {
            p->kind = PK_BSK;
            return true;
        }
    return false;
}

// Shape-aware selection (UnionSparse, Sec. I, names it without a rule; the
// thresholds are the measured ones recorded with the design). The MFMA block
// kernels wherever they run (int4: K <= 16384; fp16: K <= 4096, K % 8 == 0)
// and stage their blocks in the LDS: on every such shape both can run they
// measured faster than the split-K kernel
// (4096 x 11008 int4 N = 16: 11.2 us against 14.9 / 16.9 with 1 / 2 K
// ranges; 8192 x 8192 N = 32: 16.7 against 28.0; fp16 4096 x 4096 N = 32:
// 16.2 against 25.3). Beyond them the split-K kernel (8-24 times faster than
// the plain kernel there), with the K ranges above; fp16 with K % 8 != 0:
// the plain kernel. A forced BSP_ALGO_SPLITK takes 2 K ranges per 2-block set
// when given a workspace. Forced algorithms run their own family or return
// BSP_E_UNSUPPORTED.
int choose_plan(int dtype, const Shape &s, int64_t pbytes, int algo, bool have_ws, Plan *p) {
    *p = Plan{};
    switch (algo) {
        case BSP_ALGO_ROWWAVE:
            p->kind = PK_ROWWAVE;
            p->algo = BSP_ALGO_ROWWAVE;
            return BSP_OK;
        case BSP_ALGO_MFMA:
            return plan_mfma(dtype, s, pbytes, p) ? BSP_OK : BSP_E_UNSUPPORTED;
        case BSP_ALGO_SPLITK:
            return plan_splitk(dtype, s, pbytes, have_ws ? 2 : 1, p) ? BSP_OK : BSP_E_UNSUPPORTED;
        default:
            break;
    }
    if (s.M == 0 || s.N == 0 || s.K == 0) {
        p->kind = PK_ROWWAVE;
        return BSP_OK;
    }
    if (plan_mfma(dtype, s, pbytes, p)) {
        // The int4 ring kernel at 8 tiles per lane (K > 8192) gives way to
        // split-K (2 K ranges with a workspace) where it is at its worst:
        // - a 256-tile block too dense for the LDS (density above about
        //   0.8) would read every window from global memory, where the
        //   split-K kernel stages 64-tile chunks (4096 x 16384 at N = 8:
        //   39.6 -> 20.6 us at density 0.85, 43.6 -> 21.2 at 0.95);
        // - two column blocks (N > 16) exceed its registers (it spills 680
        //   to 824 B per lane): 4096 x 11008 at N = 32 35.7 -> 16.4 us
        //   (18.1 without a workspace), 4096 x 16384 at N = 24 45.2 -> 21.8.
        Plan sk;
        if (p->kind == PK_BT64 && !p->bt.streaming && p->bt.tpl == 8 && (p->bt.stage_bytes == 0 || p->bt.nb == 2) &&
            plan_splitk(dtype, s, pbytes, have_ws ? 2 : 1, &sk))
            *p = sk;
        return BSP_OK;
    }
    if (plan_splitk(dtype, s, pbytes, have_ws ? preferred_splits(dtype, s) : 1, p)) return BSP_OK;
    p->kind = PK_ROWWAVE;
    p->algo = BSP_ALGO_ROWWAVE;
    return BSP_OK;
}

void describe_plan(int dtype, const Plan &p, char *launch, size_t n) {
    launch[0] = 0;
    switch (p.kind) {
        case PK_BT64:
            if (p.bt.streaming)
                snprintf(launch, n, " kernel=k_bt64s_w4a4 grid=%u block=%d lds=%zu stage_kb=%d stagger=%d", p.bt.grid,
                         64 * p.bt.nwaves, p.bt.lds, p.bt.area_kb, p.bt.stagger);
            else
                snprintf(launch, n,
                         " kernel=k_bt64_w4a4 grid=%u block=%d lds=%zu tiles_per_lane=%d one_pass=%d stage_kb=%u "
                         "stage_bufs=%u stagger=%d",
                         p.bt.grid, 64 * p.bt.nwaves, p.bt.lds, p.bt.tpl, p.bt.one_pass, p.bt.stage_bytes / 1024,
                         p.bt.nbuf, p.bt.stagger);
            break;
        case PK_BT8F16:
            snprintf(launch, n, " kernel=k_bt8_f16 grid=%u block=%d lds=%zu stage_kb=%u step_slots=%d partial_ring=%d",
                     p.bf8.grid, 64 * p.bf8.nwaves, p.bf8.lds, p.bf8.area_kb, p.bf8.nstep, p.bf8.ring);
            break;
        case PK_BT64F16:
            snprintf(launch, n, " kernel=k_bt64_f16 grid=%u block=%d lds=%zu stage_kb=%u stage_bufs=%u", p.bf.grid,
                     64 * p.bf.nwaves, p.bf.lds, p.bf.stage_bytes / 1024, p.bf.nbuf);
            break;
        case PK_BSK:
            if (p.sk.streamed) {
                snprintf(launch, n, " kernel=k_bsks_w4a4 grid=%u block=%d lds=%zu blocks_per_set=%d splits=%d "
                         "tiles_per_split=%d tiles_per_lane=%d slot_kb=%d workspace=%lld", p.sk.grid, 64 * p.sk.nwaves,
                         p.sk.lds, p.sk.nbs, p.sk.S, p.sk.tps, p.sk.tpl, p.sk.iseg, (long long)p.sk.ws_bytes);
                break;
            }
            snprintf(launch, n, " kernel=k_bsk_%s grid=%u block=%d lds=%zu blocks_per_set=%d splits=%d "
                     "tiles_per_split=%d chunk_tiles=%d slot_kb=%d workspace=%lld",
                     dtype == BSP_INT4 ? "w4a4" : "f16", p.sk.grid, 64 * p.sk.nwaves, p.sk.lds, p.sk.nbs, p.sk.S,
                     p.sk.tps, (dtype == BSP_INT4 ? 8 : 4) * p.sk.nwaves, p.sk.iseg, (long long)p.sk.ws_bytes);
            break;
        default:
            snprintf(launch, n, " kernel=k_rowwave_%s", dtype == BSP_INT4 ? "w4a4" : "f16");
            break;
    }
}

// The W2A4 plan: the MFMA block kernels up to K = 16384 (2-bit values), else
// the row-wave kernel; no split-K.
int choose_plan_w2(const Shape &s, int64_t pbytes, int algo, Plan *p) {
    *p = Plan{};
    if (algo == BSP_ALGO_SPLITK) return BSP_E_UNSUPPORTED;
    if (algo != BSP_ALGO_ROWWAVE && s.K > 0 && bt64_plan(s.M, s.K, s.N, pbytes, &p->bt, 2)) {
        p->kind = PK_BT64;
        p->algo = BSP_ALGO_MFMA;
        return BSP_OK;
    }
    return algo == BSP_ALGO_MFMA ? BSP_E_UNSUPPORTED : BSP_OK;
}

int describe(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, bool have_ws, char *buf, size_t n,
             int algo = BSP_ALGO_AUTO) {
    if (dtype != BSP_INT4 && dtype != BSP_FP16 && dtype != BSP_INT2) return BSP_E_ARG;
    if (M < 0 || K < 0 || N < 0 || N > BSP_MAX_N || buf == nullptr || n == 0) return BSP_E_ARG;
    if (algo < BSP_ALGO_AUTO || algo > BSP_ALGO_SPLITK) return BSP_E_ARG;
    const Shape s{M, K, N, (K + 63) / 64, M * ((K + 63) / 64)};
    const char *dname = dtype == BSP_INT4 ? "int4" : dtype == BSP_FP16 ? "fp16" : "int2";
    // payload bytes the encoder writes for nnz nonzeros (all of W when unknown)
    const int64_t nz = nnz >= 0 ? nnz : M * K;
    const int64_t pbytes = dtype == BSP_INT4 ? (nz + 1) / 2 : dtype == BSP_FP16 ? 2 * nz : (nz + 3) / 4;
    Plan p;
    const int rc = dtype == BSP_INT2 ? choose_plan_w2(s, pbytes, algo, &p) : choose_plan(dtype, s, pbytes, algo, have_ws, &p);
    if (rc != BSP_OK) {
        snprintf(buf, n, "dtype=%s M=%lld K=%lld N=%lld nnz=%lld -> unsupported", dname, (long long)M, (long long)K,
                 (long long)N, (long long)nnz);
        return rc;
    }
    const char *name = p.algo == BSP_ALGO_ROWWAVE ? "rowwave" : p.algo == BSP_ALGO_MFMA ? "mfma" : "splitk";
    char launch[256] = "";
    if (M > 0 && N > 0) {
        describe_plan(dtype == BSP_INT2 ? BSP_INT4 : dtype, p, launch, sizeof launch);
        if (dtype == BSP_INT2) {
            // the same kernels with 2-bit values: the streaming one under its own name
            char *k = strstr(launch, "k_bt64s_w4a4");
            if (k != nullptr) memcpy(k, "k_bt64s_w2a4", 12);
            if (p.kind == PK_ROWWAVE) snprintf(launch, sizeof launch, " kernel=k_rowwave_w4a4 values=2bit");
        }
    }
    snprintf(buf, n, "dtype=%s M=%lld K=%lld N=%lld nnz=%lld -> %s%s", dname, (long long)M, (long long)K,
             (long long)N, (long long)nnz, name, launch);
    return BSP_OK;
}

// The workspace an SpMM call gets: non-null, 256-byte aligned, and at least
// what the plan needs (checked by the caller of this helper).
bool workspace_usable(const void *ws, int64_t bytes) {
    return ws != nullptr && bytes > 0 && ((uintptr_t)ws & 255u) == 0;
}

int spmm_common(int dtype, const uint64_t *bitmaps, const uint32_t *offsets, const void *payload,
                int64_t payload_bytes, int64_t M, int64_t K, const void *X, int64_t N, void *Y, void *workspace,
                int64_t workspace_bytes, int algo, hipStream_t stream) {
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, algo, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    if (workspace_bytes < 0 || (workspace == nullptr && workspace_bytes != 0)) return BSP_E_ARG;
    if (workspace != nullptr && ((uintptr_t)workspace & 255u) != 0) return BSP_E_ARG;
    const bool have_ws = workspace_usable(workspace, workspace_bytes);
    Plan p;
    rc = choose_plan(dtype, s, payload_bytes, algo, have_ws, &p);
    if (rc != BSP_OK) return rc;
    // The int4 MFMA and split-K kernels read X in whole dwords from its start
    // (the last one may reach up to 3 bytes past N * ceil(K/2), inside the
    // same page only when X starts on a 4-byte boundary); fp16 ones read
    // 16-byte pieces. An X off the boundary takes the plain kernel (automatic
    // choice) or is refused (forced).
    const bool x_aligned = ((uintptr_t)X & (dtype == BSP_INT4 ? 3u : 15u)) == 0;
    if (p.kind != PK_ROWWAVE && !x_aligned) {
        if (algo != BSP_ALGO_AUTO) return BSP_E_UNSUPPORTED;
        p = Plan{};
    }
    if (p.ws_bytes() > workspace_bytes) return BSP_E_CAPACITY;
    const uint32_t pb = (uint32_t)payload_bytes;
    switch (p.kind) {
        case PK_BT64:
            launch_bt64_w4a4(p.bt, bitmaps, offsets, (const uint8_t *)payload, pb, (int)M, (int)K, (const uint8_t *)X,
                             (int)N, (int32_t *)Y, stream);
            break;
        case PK_BT8F16:
            launch_bt8_f16(p.bf8, bitmaps, offsets, (const uint16_t *)payload, pb, (int)M, (int)K, (const uint16_t *)X,
                           (int)N, (uint16_t *)Y, stream);
            break;
        case PK_BT64F16:
            launch_bt64_f16(p.bf, bitmaps, offsets, (const uint16_t *)payload, pb, (int)M, (int)K, (const uint16_t *)X,
                            (int)N, (uint16_t *)Y, stream);
            break;
        case PK_BSK:
            launch_bsk(p.sk, sk_args(p.sk, bitmaps, offsets, payload, pb, (int)M, (int)K, X, (int)N, Y, workspace),
                       stream);
            break;
        default:
            if (dtype == BSP_INT4)
                launch_rowwave_w4a4(bitmaps, offsets, (const uint8_t *)payload, pb, (int)M, (int)K, (const uint8_t *)X,
                                    (int)N, (int32_t *)Y, stream);
            else
                launch_rowwave_f16(bitmaps, offsets, (const uint16_t *)payload, pb, (int)M, (int)K,
                                   (const uint16_t *)X, (int)N, (uint16_t *)Y, stream);
            break;
    }
    return launch_status();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the workspace of the split-K
// plans in a static device array, one copy per GPU, held until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address is handed to kernels.
#define BSP_NOALLOC_SCRATCH_BYTES ((int64_t)8 << 20)
#define BSP_NOALLOC_MAX_DEVICES 64
static __device__ __align__(256) uint8_t scratch[BSP_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex scratch_mu;
void *scratch_ptr[BSP_NOALLOC_MAX_DEVICES];   // device address of `scratch` per GPU (null: not set up)

__global__ void k_zero_scratch(uint32_t *p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The current device's scratch address, set up on its first use: the address
// of the array on that device, and the array cleared once by a fill kernel on
// `stream` (the split-K kernels need zero arrival counters; every call leaves
// them at zero again). No allocation happens.
int scratch_for_current_device(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= BSP_NOALLOC_MAX_DEVICES) return BSP_E_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return BSP_E_HIP;
        hipLaunchKernelGGL(k_zero_scratch, dim3(256), dim3(256), 0, stream, reinterpret_cast<uint32_t *>(ptr),
                           BSP_NOALLOC_SCRATCH_BYTES / 4);
        if (hipGetLastError() != hipSuccess) return BSP_E_HIP;
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return BSP_OK;
}

}  // namespace

extern "C" int spmm_bitmap_f16_noalloc(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                                       int64_t payload_bytes, int64_t M, int64_t K, const uint16_t *X, int64_t N,
                                       uint16_t *Y, int algo, hipStream_t stream) {
    // the plan spmm_bitmap_f16_ws takes with a workspace of the scratch's size
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, algo, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    Plan p;
    rc = choose_plan(BSP_FP16, s, payload_bytes, algo, true, &p);
    if (rc != BSP_OK) return rc;
    if (p.ws_bytes() > BSP_NOALLOC_SCRATCH_BYTES) return BSP_E_CAPACITY;
    void *ws = nullptr;
    if (p.ws_bytes() > 0) {
        rc = scratch_for_current_device(stream, &ws);
        if (rc != BSP_OK) return rc;
    }
    return spmm_common(BSP_FP16, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, ws,
                       ws ? BSP_NOALLOC_SCRATCH_BYTES : 0, algo, stream);
}

extern "C" int64_t bsp_noalloc_scratch_bytes(void) { return BSP_NOALLOC_SCRATCH_BYTES; }

extern "C" int bsp_select(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz) {
    if (dtype != BSP_INT4 && dtype != BSP_FP16) return -1;
    if (M < 0 || K < 0 || N < 0 || N > BSP_MAX_N) return -1;
    const Shape s{M, K, N, (K + 63) / 64, M * ((K + 63) / 64)};
    const int64_t nz = nnz >= 0 ? nnz : M * K;
    Plan p;
    choose_plan(dtype, s, dtype == BSP_INT4 ? (nz + 1) / 2 : 2 * nz, BSP_ALGO_AUTO, false, &p);
    return p.algo;
}

extern "C" int bsp_describe_selection(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, char *buf, size_t n) {
    return describe(dtype, M, K, N, nnz, false, buf, n);
}

extern "C" int bsp_describe_selection_ws(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, char *buf,
                                         size_t n) {
    return describe(dtype, M, K, N, nnz, true, buf, n);
}

extern "C" int bsp_describe_plan(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, int algo, int with_workspace,
                                 char *buf, size_t n) {
    return describe(dtype, M, K, N, nnz, with_workspace != 0, buf, n, algo);
}

extern "C" int bsp_workspace_bytes(int dtype, int64_t M, int64_t K, int64_t N, int64_t nnz, int64_t *bytes) {
    if (dtype != BSP_INT4 && dtype != BSP_FP16) return BSP_E_ARG;
    if (M < 0 || K < 0 || N < 0 || N > BSP_MAX_N || bytes == nullptr) return BSP_E_ARG;
    if (K >= BSP_MAX_K || M > INT32_MAX || M * ((K + 63) / 64) >= INT32_MAX) return BSP_E_OVERFLOW;
    const Shape s{M, K, N, (K + 63) / 64, M * ((K + 63) / 64)};
    const int64_t nz = nnz >= 0 ? nnz : M * K;
    Plan p;
    choose_plan(dtype, s, dtype == BSP_INT4 ? (nz + 1) / 2 : 2 * nz, BSP_ALGO_AUTO, true, &p);
    // the forced split-K plan may want more than the automatic one
    Plan q;
    int64_t need = p.ws_bytes();
    if (choose_plan(dtype, s, dtype == BSP_INT4 ? (nz + 1) / 2 : 2 * nz, BSP_ALGO_SPLITK, true, &q) == BSP_OK)
        need = std::max(need, q.ws_bytes());
    *bytes = need;
    return BSP_OK;
}

extern "C" int spmm_bitmap_w4a4_ws(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                   int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                                   int32_t *Y, void *workspace, int64_t workspace_bytes, int algo,
                                   hipStream_t stream) {
    return spmm_common(BSP_INT4, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, workspace, workspace_bytes,
                       algo, stream);
}

extern "C" int spmm_bitmap_w4a4_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                     int64_t payload_bytes, int64_t M, int64_t K,
                                     const uint8_t *X, int64_t N, int32_t *Y, int algo, hipStream_t stream) {
    return spmm_common(BSP_INT4, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, nullptr, 0, algo, stream);
}

extern "C" int spmm_bitmap_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                int64_t payload_bytes, int64_t M, int64_t K,
                                const uint8_t *X, int64_t N, int32_t *Y, hipStream_t stream) {
    return spmm_common(BSP_INT4, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, nullptr, 0,
                       BSP_ALGO_AUTO, stream);
}

extern "C" int spmm_bitmap_f16_ws(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                                  int64_t payload_bytes, int64_t M, int64_t K, const uint16_t *X, int64_t N,
                                  uint16_t *Y, void *workspace, int64_t workspace_bytes, int algo,
                                  hipStream_t stream) {
    return spmm_common(BSP_FP16, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, workspace, workspace_bytes,
                       algo, stream);
}

extern "C" int spmm_bitmap_f16_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                                    int64_t payload_bytes, int64_t M, int64_t K,
                                    const uint16_t *X, int64_t N, uint16_t *Y, int algo, hipStream_t stream) {
    return spmm_common(BSP_FP16, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, nullptr, 0, algo, stream);
}

extern "C" int spmm_bitmap_f16(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                               int64_t payload_bytes, int64_t M, int64_t K,
                               const uint16_t *X, int64_t N, uint16_t *Y, hipStream_t stream) {
    return spmm_common(BSP_FP16, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, nullptr, 0, BSP_ALGO_AUTO,
                       stream);
}

// ---------------------------------------------------------------------------
// Union-mask format (UnionSparse Sec. V-A, 2 x 2 areas of 16 x 64 tiles).
extern "C" int spmm_union_w4a4(const uint64_t *ubitmaps, const uint32_t *offsets, const uint64_t *rowpos,
                               const uint8_t *payload, int64_t payload_bytes, int ra, int ca, int64_t M,
                               int64_t K, const uint8_t *X, int64_t N, int32_t *Y, hipStream_t stream) {
    if (union_mask_words(ra, ca) == 0) return BSP_E_ARG;
    if (M < 0 || K < 0 || N < 0 || N > BSP_MAX_N || payload_bytes < 0) return BSP_E_ARG;
    if (payload_bytes % BSP_PAYLOAD_ALIGN != 0) return BSP_E_ARG;
    if (payload_bytes > UINT32_MAX || M > INT32_MAX) return BSP_E_OVERFLOW;
    const int64_t nlt = union_tile_count(M, K);
    if (nlt * 32 > (int64_t)UINT32_MAX) return BSP_E_OVERFLOW;    // buffer-resource ranges are 32-bit
    if (M == 0 || N == 0) return BSP_OK;
    if (Y == nullptr || offsets == nullptr) return BSP_E_ARG;
    if (K > 0 && (ubitmaps == nullptr || rowpos == nullptr || X == nullptr)) return BSP_E_ARG;
    if (payload == nullptr && payload_bytes != 0) return BSP_E_ARG;
    if (ra != 2 || ca != 2) return BSP_E_UNSUPPORTED;
    if (K > BSP_UNION_MAX_K) return BSP_E_UNSUPPORTED;
    if (K == 0) {
        const int64_t n = M * N;
        hipLaunchKernelGGL(k_ie_zero, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 1024)), dim3(256), 0, stream,
                           Y, n);
        return launch_status();
    }
    if (((uintptr_t)X & 3u) != 0) return BSP_E_UNSUPPORTED;
    IePlan p;
    if (!ie_plan(M, K, N, &p)) return BSP_E_UNSUPPORTED;
    launch_ie_w4a4(p, offsets, ubitmaps, rowpos, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, Y,
                   stream);
    return launch_status();
}

// ---------------------------------------------------------------------------
// Dequant epilogue and grouped launch (int4 MFMA kernels).

__global__ void k_f16_zero(uint16_t *__restrict__ Y, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) Y[i] = 0;
}

__global__ void k_dq_zero(uint16_t *__restrict__ Yh, const float *__restrict__ sw, const float *__restrict__ sx,
                          int64_t M, int64_t N) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M * N; i += (int64_t)gridDim.x * blockDim.x)
        Yh[i] = bt_dequant(0, sw[i % M], sx[i / M]);
}

extern "C" int spmm_bitmap_w4a4_dq(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                   int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                                   const float *scale_w, const float *scale_x, uint16_t *Yh, hipStream_t stream) {
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Yh, BSP_ALGO_AUTO, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    if (scale_w == nullptr || scale_x == nullptr) return BSP_E_ARG;
    if (K == 0) {
        const int64_t n = M * N;
        hipLaunchKernelGGL(k_dq_zero, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 1024)), dim3(256), 0, stream,
                           Yh, scale_w, scale_x, M, N);
        return launch_status();
    }
    Plan p;
    rc = choose_plan(BSP_INT4, s, payload_bytes, BSP_ALGO_MFMA, false, &p);
    if (rc != BSP_OK || p.kind != PK_BT64) return BSP_E_UNSUPPORTED;
    if (((uintptr_t)X & 3u) != 0) return BSP_E_UNSUPPORTED;
    launch_bt64_w4a4(p.bt, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, nullptr,
                     stream, BtEpi{Yh, scale_w, scale_x});
    return launch_status();
}

namespace {

// The streaming plan of one item of a grouped launch with `grid` workgroups
// (at most nblk_cap blocks each).
bool bts_item_plan(int64_t M, int64_t K, int64_t N, int64_t pbytes, int64_t grid, int nblk_cap, BtPlan *p) {
    if (!bt64_plan(M, K, N, pbytes, p) || !p->streaming) return false;
    const int64_t blocks = (M + BT_ROWS - 1) / BT_ROWS;
    grid = std::max<int64_t>(grid, (blocks + nblk_cap - 1) / nblk_cap);
    grid = std::min<int64_t>(grid, blocks);
    p->grid = (unsigned)grid;
    p->bq = (int)(blocks / grid);
    p->br = (int)(blocks % grid);
    return true;
}

}  // namespace

extern "C" int spmm_bitmap_w4a4_grouped(const bsp_w4a4_item *items, int count, int64_t K, hipStream_t stream) {
    if (items == nullptr || count < 1 || count > BSP_GROUP_MAX) return BSP_E_ARG;
    if (K < 0) return BSP_E_ARG;
    int64_t total_blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bsp_w4a4_item &it = items[i];
        Shape s;
        const void *y = it.Yh != nullptr ? (const void *)it.Yh : (const void *)it.Y;
        int rc = check_args(it.bitmaps, it.offsets, it.payload, it.payload_bytes, it.M, K, it.X, it.N, y,
                            BSP_ALGO_AUTO, &s);
        if (rc != BSP_OK) return rc;
        if (it.M == 0 || it.N == 0) continue;
        if ((it.Y != nullptr) == (it.Yh != nullptr)) return BSP_E_ARG;   // exactly one output
        if (it.Yh != nullptr && (it.scale_w == nullptr || it.scale_x == nullptr)) return BSP_E_ARG;
        if (((uintptr_t)it.X & 3u) != 0) return BSP_E_UNSUPPORTED;
        total_blocks += (it.M + BT_ROWS - 1) / BT_ROWS;
    }
    if (total_blocks == 0) return BSP_OK;
    if (K == 0) return BSP_E_UNSUPPORTED;
    BtsGroup g{};
    g.K = (int)K;
    int nb = 1, d = 2, nwaves = 0;
    size_t lds = 0;
    int64_t wg = 0;
    BtPlan plans[BSP_GROUP_MAX];
    int idx[BSP_GROUP_MAX], n_items = 0;
    // up to BTS_GROUP_NBLK blocks per workgroup, so that the group fits in
    // one round of workgroups; three (the plain kernel's) when four do not
    // fit in LDS
    for (int cap = BTS_GROUP_NBLK; cap >= BTS_NBLK; --cap) {
        nb = 1, d = 2, nwaves = 0, lds = 0, wg = 0, n_items = 0;
        for (int i = 0; i < count; ++i) {
            const bsp_w4a4_item &it = items[i];
            if (it.M == 0 || it.N == 0) continue;
            const int64_t blocks = (it.M + BT_ROWS - 1) / BT_ROWS;
            // the CUs are shared out in proportion to the items' row blocks
            const int64_t share = std::max<int64_t>(1, BT_CUS * blocks / total_blocks);
            if (!bts_item_plan(it.M, K, it.N, it.payload_bytes, share, cap, &plans[n_items])) return BSP_E_UNSUPPORTED;
            nb = std::max(nb, plans[n_items].nb);
            d = std::max(d, plans[n_items].streaming);
            nwaves = plans[n_items].nwaves;
            idx[n_items++] = i;
        }
        for (int j = 0; j < n_items; ++j) {
            const BtPlan &p = plans[j];
            lds = std::max(lds, bts_lds(nwaves, nb, p.area_kb, p.bq + (p.br > 0 ? 1 : 0), BTS_GROUP_NBLK));
        }
        if (lds <= (size_t)BT_LDS_MAX) break;
    }
    for (int j = 0; j < n_items; ++j) {
        const BtPlan &p = plans[j];
        const bsp_w4a4_item &it = items[idx[j]];
        BtsItem &b = g.item[j];
        b.offsets = it.offsets;
        b.bitmaps = it.bitmaps;
        b.X = it.X;
        b.payload = it.payload;
        b.Y = it.Y;
        b.Yh = it.Yh;
        b.sw = it.scale_w;
        b.sx = it.scale_x;
        b.M = (int)it.M;
        b.N = (int)it.N;
        b.bq = p.bq;
        b.br = p.br;
        b.wg_begin = (int)wg;
        b.payload_bytes = (uint32_t)it.payload_bytes;
        b.stagger = (uint32_t)p.stagger;
        b.area_kb = (uint32_t)p.area_kb;
        wg += p.grid;
    }
    if (lds > (size_t)BT_LDS_MAX || wg > INT32_MAX) return BSP_E_UNSUPPORTED;
    g.count = n_items;
    if (K % 8 == 0)
        launch_bts_group_x<false>(g, nb, d, (unsigned)wg, nwaves, lds, stream);
    else
        launch_bts_group_x<true>(g, nb, d, (unsigned)wg, nwaves, lds, stream);
    return launch_status();
}

// ---------------------------------------------------------------------------
// W2A4: 2-bit weights in the BT64 format, int4 activations, int32 Y.
extern "C" int spmm_bitmap_w2a4_algo(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                     int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N,
                                     int32_t *Y, int algo, hipStream_t stream) {
    Shape s;
    int rc = check_args(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, algo, &s);
    if (rc != BSP_OK || M == 0 || N == 0) return rc;
    // the MFMA block kernels (streaming up to K = 4096, ring up to 16384),
    // else the row-wave kernel
    Plan p;
    rc = choose_plan_w2(s, payload_bytes, algo, &p);
    if (rc != BSP_OK) return rc;
    if (p.kind == PK_BT64 && ((uintptr_t)X & 3u) != 0) {
        if (algo == BSP_ALGO_MFMA) return BSP_E_UNSUPPORTED;
        p.kind = PK_ROWWAVE;
    }
    const BtPlan &bp = p.bt;
    if (p.kind == PK_BT64) {
        if (bp.streaming)
            launch_bt64s_w2a4(bp, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, Y,
                              stream);
        else
            launch_bt64_w2a4(bp, bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, Y,
                             stream);
    } else {
        launch_rowwave_w4a4<2>(bitmaps, offsets, payload, (uint32_t)payload_bytes, (int)M, (int)K, X, (int)N, Y, stream);
    }
    return launch_status();
}

extern "C" int spmm_bitmap_w2a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                int64_t payload_bytes, int64_t M, int64_t K, const uint8_t *X, int64_t N, int32_t *Y,
                                hipStream_t stream) {
    return spmm_bitmap_w2a4_algo(bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, BSP_ALGO_AUTO, stream);
}

// ---------------------------------------------------------------------------
// Tiled-CBC product with dynamic activation pruning (fp16).
extern "C" int spmspv_cbc_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t *bytes) {
    if (bytes == nullptr || M < 0 || K < 0 || N < 0 || N > BSP_CBC_MAX_N) return BSP_E_ARG;
    *bytes = (M == 0 || K == 0 || N == 0) ? 0 : cbc_plan(M, K, N, true).ws_bytes;
    return BSP_OK;
}

extern "C" int spmspv_cbc_f16(const uint32_t *tile_offsets, const uint32_t *colinfo, const uint64_t *bitmaps,
                              const uint16_t *values, int64_t values_bytes, int64_t M, int64_t K, const uint16_t *X,
                              int64_t N, float threshold, uint16_t *Y, void *workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
    if (M < 0 || K < 0 || N < 0 || N > BSP_CBC_MAX_N || values_bytes < 0 || workspace_bytes < 0) return BSP_E_ARG;
    if (!(threshold >= 0.f) || std::isinf(threshold)) return BSP_E_ARG;     // NaN, negative or infinite
    if (values_bytes % BSP_PAYLOAD_ALIGN != 0) return BSP_E_ARG;
    if (values_bytes > UINT32_MAX || M > INT32_MAX || K > INT32_MAX) return BSP_E_OVERFLOW;
    if (workspace == nullptr && workspace_bytes != 0) return BSP_E_ARG;
    if (workspace != nullptr && ((uintptr_t)workspace & 255u) != 0) return BSP_E_ARG;
    if (M == 0 || N == 0) return BSP_OK;
    if (Y == nullptr || tile_offsets == nullptr) return BSP_E_ARG;
    if (K > 0 && (colinfo == nullptr || bitmaps == nullptr || X == nullptr)) return BSP_E_ARG;
    if (values == nullptr && values_bytes != 0) return BSP_E_ARG;
    if (cbc_gtile_count(M, K) * BSP_CBC_TILE_K * (BSP_CBC_TILE_M / 64) * 8 > (int64_t)INT32_MAX * 4) return BSP_E_OVERFLOW;
    if (K == 0) {
        const int64_t n = M * N;
        hipLaunchKernelGGL(k_f16_zero, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 1024)), dim3(256), 0, stream,
                           Y, n);
        return launch_status();
    }
    const bool split = workspace != nullptr && workspace_bytes > 0;
    const CbcPlan p = cbc_plan(M, K, N, split);
    if (p.ws_bytes > workspace_bytes) return BSP_E_CAPACITY;
    float *part = p.S > 1 ? (float *)((uint8_t *)workspace + CBC_WS_COUNTERS) : nullptr;
    uint32_t *cnt = p.S > 1 ? (uint32_t *)workspace : nullptr;
    const unsigned grid = (unsigned)((int64_t)p.bands * p.S);
    // the instance with the fewest activation columns that holds N
#define CBC_LAUNCH(NM)                                                                                              \
    hipLaunchKernelGGL(k_cbc_f16<NM>, dim3(grid), dim3(1024), 0, stream, tile_offsets, colinfo, bitmaps, values,   \
                       (uint32_t)values_bytes, (int)M, (int)K, X, (int)N, threshold, Y, part, cnt, p.S, p.G)
    if (N == 1)
        CBC_LAUNCH(1);
    else if (N == 2)
        CBC_LAUNCH(2);
    else if (N <= 4)
        CBC_LAUNCH(4);
    else
        CBC_LAUNCH(CBC_NMAX);
#undef CBC_LAUNCH
    return launch_status();
}
