// kernels_mfma_wg.hip -- MFMA kernel with workgroup-contiguous staging (gfx950).
//
// Same decode and contraction as kernels_mfma.hip (lane-per-tile selector /
// v_perm decode into x16 int8, v_mfma_i32_16x16x64_i8), but the staging is
// organised around a property of the stream: the payload of 16 consecutive
// rows is ONE contiguous byte range, [offsets[m0*T], offsets[(m0+16)*T]).
// The workgroup therefore needs only those two offsets before it can request
// its whole payload, and it requests it with fully coalesced LDS DMA (each
// instruction moves 1 KB of consecutive bytes, i.e. whole cache lines),
// instead of one short range per row and chunk. When the whole of X fits the
// workgroup's LDS budget it is staged the same way, once per workgroup, and
// each lane reads its slab from LDS (with a zero row for columns n >= N).
//
// LDS layout: [selector table 2 KB][X area][payload area]; the payload area
// is sized for the densest possible 16-row block (16 x T tiles x 32 bytes).
// The four-plus wavefronts split K in 16-tile chunks exactly as in
// kernels_mfma.hip and are summed through LDS at the end.

template <int NBLK, bool XLDS>
__global__ __launch_bounds__(BSP_WAVE * BSP_MF_MAX_WAVES) void k_mfma_wg_w4a4(
        const uint64_t *__restrict__ bitmaps, const uint32_t *__restrict__ offsets,
        const uint8_t *__restrict__ payload, uint32_t payload_bytes, int M, int K,
        const uint8_t *__restrict__ X, int N, int32_t *__restrict__ Y,
        uint32_t x_area_bytes, uint32_t pay_area_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t bsp_smem[];
    const int nwaves = blockDim.x / BSP_WAVE;
    const int wave = threadIdx.x / BSP_WAVE;
    const int lane = threadIdx.x % BSP_WAVE;
    const uint2 *lut = reinterpret_cast<const uint2 *>(bsp_smem);
    uint8_t *x_area = bsp_smem + BSP_MF_LUT_BYTES;
    uint8_t *pay_area = x_area + x_area_bytes;

    const int T = (K + 63) >> 6;
    const int m0 = blockIdx.x * BSP_MF_ROWS;
    const int rows = min(BSP_MF_ROWS, M - m0);
    const int r = lane & 15, s = lane >> 4;
    const int m = m0 + r;
    const bool row_ok = r < rows;
    const int64_t rowg = (int64_t)(m0 + min(r, rows - 1)) * T;
    const int xs = (K + 1) >> 1;     // X row stride in bytes (K % 8 == 0 on this path)
    const __amdgpu_buffer_rsrc_t prs = bsp_rsrc(payload, payload_bytes);
    const __amdgpu_buffer_rsrc_t xrs = bsp_rsrc(X, (uint32_t)(N * xs));

    // (1) The block's payload range: two offsets, the only loads the payload waits on.
    const uint32_t nibA = offsets[(int64_t)m0 * T];
    const uint32_t nibB = offsets[(int64_t)(m0 + rows) * T];

    // (2) Selector table and X by DMA (no dependency on the offsets).
    {
        const __amdgpu_buffer_rsrc_t lrs = bsp_rsrc(&bsp_mf_lut_global, (uint32_t)sizeof(BspMfLut));
        constexpr int lut_units = BSP_MF_LUT_BYTES / 16;
        for (int u0 = wave * BSP_WAVE; u0 < lut_units; u0 += nwaves * BSP_WAVE)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (bsp_lds_void *)(bsp_smem + u0 * 16), 16, lane * 16,
                                                     u0 * 16, 0, 0);
    }
    // X rows sit xsl = xs + 16 bytes apart in LDS so that the 16 MFMA columns
    // (lanes reading the same tile of different rows) start in different banks.
    const int xsl = xs + 16;
    if (XLDS) {
        const int row_units = xs / 16;              // xs is a multiple of 16 on this path
        const int pieces = (row_units + BSP_WAVE - 1) / BSP_WAVE;
        for (int job = wave; job < N * pieces; job += nwaves) {
            const int n = job / pieces, u0 = (job % pieces) * BSP_WAVE;
            if (u0 + lane < row_units)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (bsp_lds_void *)(x_area + n * xsl + u0 * 16), 16,
                                                         lane * 16, (n * xs + u0 * 16), 0, 0);
        }
        // a zero row after X for the MFMA columns n >= N
        bsp_v4i *zero_row = reinterpret_cast<bsp_v4i *>(x_area + N * xsl);
        for (int u = (int)threadIdx.x; u < xsl / 16; u += (int)blockDim.x) zero_row[u] = bsp_v4i{0, 0, 0, 0};
    }

    // (3) The payload: one contiguous range, moved 1 KB per wavefront instruction.
    const uint32_t uA = nibA >> 5;                       // first 16-byte unit of the block
    const uint32_t uB = (nibB >> 5) + 2u;                // +1 past the end, +1 for the last window
    // never more than the area holds, whatever the offsets say
    const uint32_t nunits = uB > uA ? min(uB - uA, pay_area_bytes / 16u) : 0u;
    for (uint32_t u0 = (uint32_t)(wave * BSP_WAVE); u0 < nunits; u0 += (uint32_t)(nwaves * BSP_WAVE))
        if (u0 + (uint32_t)lane < nunits)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bsp_lds_void *)(pay_area + u0 * 16), 16, lane * 16,
                                                     (int)((uA + u0) * 16), 0, 0);

    bsp_v4i acc[NBLK];
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) acc[nb] = bsp_v4i{0, 0, 0, 0};
    const uint32_t pay_nib = (uint32_t)(uintptr_t)(const bsp_lds_void *)pay_area * 2u - (uA << 5);
    bool staged = false;

    for (int c0 = wave * BSP_MF_CHUNK; c0 < T || !staged; c0 += nwaves * BSP_MF_CHUNK) {
        const bool live = c0 < T;
        const int c1 = min(T, c0 + BSP_MF_CHUNK);
        const int ts0 = min(c1, c0 + s * BSP_MF_TPL), ts1 = min(c1, ts0 + BSP_MF_TPL);
        // (4) this lane's start position and words (global, 16 rows x 32 bytes per instruction)
        uint32_t lane_nib0 = nibA;
        uint64_t words[BSP_MF_TPL];
        if (live && row_ok) lane_nib0 = offsets[rowg + min(ts0, c1)];
#pragma unroll
        for (int i = 0; i < BSP_MF_TPL; ++i)
            words[i] = (live && row_ok && ts0 + i < ts1) ? bitmaps[rowg + ts0 + i] : 0ull;
        uint32_t xd[BSP_MF_TPL][NBLK][8];
        if (!XLDS) {
#pragma unroll
            for (int i = 0; i < BSP_MF_TPL; ++i)
#pragma unroll
                for (int nb = 0; nb < NBLK; ++nb) {
                    // column n >= N reads past N*xs: the range check returns zeros
                    const uint32_t off = (uint32_t)((r + 16 * nb) * xs + (ts0 + i) * 32);
                    const bsp_v4i v0 = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
                    const bsp_v4i v1 = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16, 0, 0));
                    xd[i][nb][0] = v0.x; xd[i][nb][1] = v0.y; xd[i][nb][2] = v0.z; xd[i][nb][3] = v0.w;
                    xd[i][nb][4] = v1.x; xd[i][nb][5] = v1.y; xd[i][nb][6] = v1.z; xd[i][nb][7] = v1.w;
                }
        }
        if (!staged) {   // every wavefront's DMA must have landed before anyone reads
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            staged = true;
        }
        if (!live) break;
        if (XLDS) {
#pragma unroll
            for (int i = 0; i < BSP_MF_TPL; ++i)
#pragma unroll
                for (int nb = 0; nb < NBLK; ++nb) {
                    const int n = min(r + 16 * nb, N);          // row N of the X area is zero
                    const bsp_v4i *src = reinterpret_cast<const bsp_v4i *>(x_area + n * xsl + (ts0 + i) * 32);
                    const bsp_v4i v0 = src[0], v1 = src[1];
                    xd[i][nb][0] = v0.x; xd[i][nb][1] = v0.y; xd[i][nb][2] = v0.z; xd[i][nb][3] = v0.w;
                    xd[i][nb][4] = v1.x; xd[i][nb][5] = v1.y; xd[i][nb][6] = v1.z; xd[i][nb][7] = v1.w;
                }
        }
        uint32_t q = pay_nib + lane_nib0;
#pragma unroll
        for (int i = 0; i < BSP_MF_TPL; ++i) {
            BspMfFetch f;
            bsp_mf_fetch(words[i], q, lut, f);
            q += __builtin_popcountll(words[i]);
            uint32_t A[16];
            bsp_mf_build(f, A);
#pragma unroll
            for (int nb = 0; nb < NBLK; ++nb) {
                uint32_t B[16];
                bsp_mf_convert_x(xd[i][nb], B);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bsp_v4i a = {(int)A[4 * k], (int)A[4 * k + 1], (int)A[4 * k + 2], (int)A[4 * k + 3]};
                    const bsp_v4i b = {(int)B[4 * k], (int)B[4 * k + 1], (int)B[4 * k + 2], (int)B[4 * k + 3]};
                    acc[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[nb], 0, 0, 0);
                }
            }
        }
    }

    // --- reduce the wavefronts' K chunks through LDS, then write Y (x256 removed)
    __syncthreads();
    int32_t *red = reinterpret_cast<int32_t *>(pay_area);
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((wave * NBLK + nb) * 4 + i) * BSP_WAVE + lane] = acc[nb][i];
    __syncthreads();
    // D layout of v_mfma_i32_16x16x64_i8: lane l, register i -> row 4*(l/16)+i, column l%16.
    for (int o = threadIdx.x; o < NBLK * 256; o += blockDim.x) {
        const int nb = o >> 8, col = (o >> 4) & 15, rl = o & 15;   // consecutive threads -> consecutive rows
        const int ln = (rl >> 2) * 16 + col, i = rl & 3;
        int32_t sum = 0;
        for (int w = 0; w < nwaves; ++w) sum += red[((w * NBLK + nb) * 4 + i) * BSP_WAVE + ln];
        const int n = col + 16 * nb, mm = m0 + rl;
        if (n < N && mm < M) Y[(int64_t)n * M + mm] = sum >> 8;
    }
}

// Launch plan of the workgroup-contiguous kernel: false when the densest
// 16-row block would not fit in LDS (very long K).
struct BspMfWgPlan {
    int nwaves;
    uint32_t x_area, pay_area;
    size_t lds;
    bool x_in_lds;
};

static bool mfma_wg_plan(int M, int K, int N, BspMfWgPlan *p) {
    const int T = (K + 63) / 64;
    const int xs = (K + 1) / 2;
    p->nwaves = std::max(1, std::min(BSP_MF_MAX_WAVES, (T + BSP_MF_CHUNK - 1) / BSP_MF_CHUNK));
    const int nblk = N <= 16 ? 1 : 2;
    const size_t red = (size_t)p->nwaves * nblk * 4 * BSP_WAVE * 4;
    p->pay_area = (uint32_t)std::max<size_t>((size_t)(32 * T + 3) * 16, red);
    const size_t lds_max = 160 * 1024;
    const size_t base = BSP_MF_LUT_BYTES + p->pay_area;
    if (base > lds_max) return false;
    // Stage X when it fits in the LDS share each workgroup can have while the
    // whole grid stays resident in one round (workgroups per CU on 256 CUs).
    const int wgs = (M + BSP_MF_ROWS - 1) / BSP_MF_ROWS;
    const int per_cu = std::max(1, (wgs + 255) / 256);
    const size_t budget = lds_max / per_cu;
    const size_t x_bytes = (size_t)(N + 1) * (xs + 16);     // X and one zero row, padded rows
    p->x_in_lds = xs % 16 == 0 && base + x_bytes <= budget;
    p->x_area = p->x_in_lds ? (uint32_t)((x_bytes + 15) / 16 * 16) : 0u;
    p->lds = base + p->x_area;
    return true;
}

template <int NBLK>
static void launch_mfma_wg_nb(const BspMfWgPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                              const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                              int32_t *Y, hipStream_t stream) {
    const dim3 block(BSP_WAVE * p.nwaves), grid((unsigned)((M + BSP_MF_ROWS - 1) / BSP_MF_ROWS));
    if (p.x_in_lds) {
        hipFuncSetAttribute((const void *)k_mfma_wg_w4a4<NBLK, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds);
        hipLaunchKernelGGL((k_mfma_wg_w4a4<NBLK, true>), grid, block, p.lds, stream, bitmaps, offsets, payload,
                           payload_bytes, M, K, X, N, Y, p.x_area, p.pay_area);
    } else {
        hipFuncSetAttribute((const void *)k_mfma_wg_w4a4<NBLK, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.lds);
        hipLaunchKernelGGL((k_mfma_wg_w4a4<NBLK, false>), grid, block, p.lds, stream, bitmaps, offsets, payload,
                           payload_bytes, M, K, X, N, Y, p.x_area, p.pay_area);
    }
}
