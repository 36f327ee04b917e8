// kernels_union.hip -- int4 x int4 -> int32 SpMM over the union-mask (IE-BME)
// format on gfx950 (CDNA4): UnionSparse, Sec. V-A ("IE-BME Representation",
// Fig. 7) with 16 x 64 local tiles split into 2 x 2 areas of 8 x 32, rows of
// each tile optionally reordered offline (Sec. V-B).
//
// Format, per local tile (LT) t in row-major order over the matrix: four
// 64-bit union-mask words (logical row i of the 8 x 32 mask is dword i of the
// tile's 32 bytes, leftmost position in bit 0), the value offset o_t, a rowpos
// word (nibble r = reordered position of tile row r) and 4 P_t int4 values,
// area q's stream at o_t + q P_t (q = 2 a + c: area row a, area column c).
//
// Work split. A workgroup of 8 wavefronts owns up to IE_MAXB consecutive row
// bands (16 rows each); wavefront w owns tile columns [w L, (w+1) L) of each,
// L = ceil(T / 8). Its work is a sequence of steps, band by band, each a chunk
// of up to 8 consecutive LTs of one band: their masks, rowpos words and
// offsets come in as one dword per lane, their payload (one contiguous
// stretch of the value array, at most 8 x 512 bytes) by LDS DMA into one of
// the wavefront's two slots, and their X columns as 16-byte granules, all
// issued one step ahead. Slots, tables and X are private to the wavefront, so
// no step waits at a barrier; the per-band partial sums meet in LDS at the end
// of each band (integer adds, exact in any order).
//
// MFMA mapping. An LT is the A operand of one v_mfma_i32_16x16x64_i8 per 16
// columns of X. Lane l = R + 16 kg holds tile row R in its original order and
// the 16 columns {8 kg .. 8 kg + 7} and {32 + 8 kg .. 32 + 8 kg + 7}. Row R
// sits at reordered position p = rowpos[R]: area row a = p >> 3, logical row
// g = p & 7. Its 16 values are logical byte kg of mask row g, read from the
// streams of areas (a, 0) and (a, 1) at one rank, so the lane makes one
// selector-table lookup and two payload-window reads. The B operand has the
// same column order: X dwords kg and 4 + kg of the tile's 32-byte X segment,
// which a 4 x 4 transpose over the lane groups delivers from one 16-byte
// load per lane per two LTs.
//
// Values are decoded in the x16 form (a nibble in the high half of a byte,
// as the BT64 kernels do), so products are 256 w x and every wavefront's
// partial is shifted right by 8 (exact) before the partials are added. With K
// at most IE_MAX_K no int32 sum can overflow: 256 * 64 * K < 2^31.

#define IE_WAVES 8
#define IE_CHUNK 8                    // LTs per step
#define IE_MAXB 4                     // row bands per workgroup
#define IE_SLOT_KB 5                  // DMA instructions (1 KB each) per slot: 8 x 512 B + alignment
#define IE_SLOT_BYTES (IE_SLOT_KB * 1024)
#define IE_META_BYTES 512             // per wavefront: 64 x (mask row, rows-before count)
#define IE_SUMS_BYTES (IE_MAXB * 32 * 16 * 4)
#define IE_LDS_BYTES (IE_SUMS_BYTES + BT_LUT_BYTES + IE_WAVES * IE_META_BYTES + IE_WAVES * 2 * IE_SLOT_BYTES)
#define IE_MAX_K BSP_UNION_MAX_K
#define IE_OOR 0xFFFFFFF0u            // a buffer offset past every range: reads zeros

// Two dwords of a slot holding nibbles pos .. pos + 7 (pos counted from the
// slot's start), aligned by a funnel shift.
__device__ __forceinline__ uint32_t ie_window(uint32_t slot_addr, uint32_t pos) {
    const bt_lds_u32 *q = (const bt_lds_u32 *)(uintptr_t)(slot_addr + ((pos >> 1) & ~3u));
    return __builtin_amdgcn_alignbit(q[1], q[0], (pos & 7u) << 2);
}

// A operand dwords of one window: {even ranks, odd ranks} placed by the
// byte's selector pair.
__device__ __forceinline__ void ie_place(uint32_t w, uint2 sel, uint32_t &d0, uint32_t &d1) {
    const uint32_t s_odd = w & 0xF0F0F0F0u;
    const uint32_t s_even = (w << 4) & 0xF0F0F0F0u;
    d0 = __builtin_amdgcn_perm(s_odd, s_even, sel.x);
    d1 = __builtin_amdgcn_perm(s_odd, s_even, sel.y);
}

// The 4 x 4 dword transpose over lane groups (lanes kg*16 .. kg*16+15): group
// kg's element d goes to group d's element kg. Every lane must be active.
__device__ __forceinline__ bt_v4i ie_transpose(bt_v4i v) {
    auto a = __builtin_amdgcn_permlane32_swap((unsigned)v.x, (unsigned)v.z, false, false);
    auto b = __builtin_amdgcn_permlane32_swap((unsigned)v.y, (unsigned)v.w, false, false);
    auto c = __builtin_amdgcn_permlane16_swap((unsigned)a[0], (unsigned)b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap((unsigned)a[1], (unsigned)b[1], false, false);
    return bt_v4i{(int)c[0], (int)c[1], (int)d[0], (int)d[1]};
}

template <int NCH, bool XU>
__global__ __launch_bounds__(IE_WAVES * 64) void k_ie_w4a4(
        const uint32_t *__restrict__ offsets, const uint64_t *__restrict__ ubitmaps,
        const uint64_t *__restrict__ rowpos, const uint8_t *__restrict__ payload, uint32_t payload_bytes,
        int M, int K, int bq, int br, const uint8_t *__restrict__ X, int N, int32_t *__restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ie_smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int R = lane & 15, kg = lane >> 4;
    const int T = (K + 63) >> 6;
    const int bands = (M + 15) >> 4;
    const int gid = (int)blockIdx.x;
    const int b0 = gid * bq + min(gid, br);
    const int nb = bq + (gid < br ? 1 : 0);            // 1 .. IE_MAXB
    const int L = (T + IE_WAVES - 1) / IE_WAVES;
    const int c0 = wave * L, c1 = min(T, c0 + L);
    const int nck = c1 > c0 ? (c1 - c0 + IE_CHUNK - 1) / IE_CHUNK : 0;
    const int S = nb * nck;                            // steps of this wavefront
    const uint32_t xs = ((uint32_t)K + 1u) >> 1;
    const uint32_t nlt = (uint32_t)bands * (uint32_t)T;

    int32_t *sums = reinterpret_cast<int32_t *>(ie_smem);   // [IE_MAXB][32 columns][16 rows]
    uint8_t *lut8 = ie_smem + IE_SUMS_BYTES;
    uint8_t *meta8 = lut8 + BT_LUT_BYTES + wave * IE_META_BYTES;
    uint8_t *slot8 = lut8 + BT_LUT_BYTES + IE_WAVES * IE_META_BYTES + wave * 2 * IE_SLOT_BYTES;
    const uint32_t lut_base = bt_lds_addr(lut8) + (uint32_t)(lane % BT_LUT_COPIES) * 8u;
    const uint32_t meta_addr = bt_lds_addr(meta8);
    const uint32_t slot_addr0 = bt_lds_addr(slot8);

    const __amdgpu_buffer_rsrc_t ors = bt_rsrc(offsets, (nlt + 1u) * 4u);
    const __amdgpu_buffer_rsrc_t urs = bt_rsrc(ubitmaps, nlt * 32u);
    const __amdgpu_buffer_rsrc_t rrs = bt_rsrc(rowpos, nlt * 8u);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(payload, payload_bytes);
    const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(X, bt_x_range(N, xs));

    // chunk boundaries of every step: lane j = bi (nck + 1) + ci holds the
    // value offset of tile column min(c1, c0 + 8 ci) of band b0 + bi
    uint32_t bnd = 0;
    {
        const int j = lane, per = nck + 1;
        uint32_t off = IE_OOR;
        if (nck > 0 && j < nb * per) {
            const int bi = j / per, ci = j - bi * per;
            const uint32_t t = (uint32_t)(b0 + bi) * (uint32_t)T + (uint32_t)min(c1, c0 + IE_CHUNK * ci);
            off = t * 4u;
        }
        bnd = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ors, off, 0, 0);
    }
    uint32_t issued = 1;

    for (int o = threadIdx.x; o < IE_MAXB * 32 * 16; o += blockDim.x) sums[o] = 0;
    for (int e = threadIdx.x; e < 256 * BT_LUT_COPIES; e += blockDim.x) {
        const uint2 v = bt_lut_entry((uint32_t)e / BT_LUT_COPIES);
        *reinterpret_cast<uint2 *>(lut8 + (size_t)e * 8) = v;
    }
    __syncthreads();

    uint32_t maskv[2], rpv[2], offv[2], g0s[2], mark[2] = {0, 0};
    bt_v4i xg[2][NCH][4];

    // Issue the loads of step s into slot k. A step past the last one issues
    // the same instructions with every offset out of range (they read zeros
    // and move no data): the count per step is then fixed, so every wait
    // below is exact.
    auto issue = [&](int s, int k) {
        const bool live = s < S;
        const int bi = live ? s / nck : 0, ci = live ? s - bi * nck : 0;
        const int band = b0 + bi;
        const int cc0 = c0 + IE_CHUNK * ci;
        const int n_lt = live ? min(IE_CHUNK, c1 - cc0) : 0;
        const uint32_t t0 = (uint32_t)band * (uint32_t)T + (uint32_t)cc0;
        const int jb = bi * (nck + 1) + ci;
        const uint32_t oa = live ? (uint32_t)__builtin_amdgcn_readlane((int)bnd, jb) : 0u;
        const uint32_t ob = live ? (uint32_t)__builtin_amdgcn_readlane((int)bnd, jb + 1) : 0u;
        maskv[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                urs, lane < 8 * n_lt ? t0 * 32u + 4u * (uint32_t)lane : IE_OOR, 0, 0);
        rpv[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                rrs, lane < 2 * n_lt ? t0 * 8u + 4u * (uint32_t)lane : IE_OOR, 0, 0);
        offv[k] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                ors, lane <= n_lt && live ? (t0 + (uint32_t)lane) * 4u : IE_OOR, 0, 0);
        // X: granule kg of the 64-byte segment of LT pair j (column R + 16 nch)
#pragma unroll
        for (int nch = 0; nch < NCH; ++nch) {
            const int n = R + 16 * nch;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = cc0 + 2 * j + (kg >> 1);
                const bool ok = live && n < N && col < c1;
                const uint32_t off = ok ? (uint32_t)n * xs + (uint32_t)(cc0 + 2 * j) * 32u + 16u * (uint32_t)kg
                                        : IE_OOR;
                xg[k][nch][j] = bt_load_x16<XU>(xrs, off);
            }
        }
        // payload of the chunk: granules [G0, G1), at most IE_SLOT_KB x 64 of them
        const uint32_t G0 = oa >> 5, G1 = live ? (ob + 31u) >> 5 : 0u;
        const uint32_t dst = slot_addr0 + (uint32_t)k * IE_SLOT_BYTES;
#pragma unroll
        for (int i = 0; i < IE_SLOT_KB; ++i) {
            const uint32_t gr = G0 + 64u * (uint32_t)i + (uint32_t)lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(uintptr_t)(dst + 1024u * (uint32_t)i), 16,
                                                     gr < G1 ? gr * 16u : IE_OOR, 0, 0, BT_NT);
        }
        g0s[k] = G0;
        issued += 3u + (uint32_t)(NCH * 4 * (XU ? 2 : 1)) + (uint32_t)IE_SLOT_KB;
        mark[k] = issued;
    };

    bt_v4i acc[NCH], accb[IE_MAXB][NCH];
#pragma unroll
    for (int nch = 0; nch < NCH; ++nch) {
        acc[nch] = bt_v4i{0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < IE_MAXB; ++b) accb[b][nch] = bt_v4i{0, 0, 0, 0};
    }

    auto process = [&](int s, int k) {
        const int bi = s / nck, ci = s - bi * nck;
        const int cc0 = c0 + IE_CHUNK * ci;
        const int n_lt = min(IE_CHUNK, c1 - cc0);
        bt_wait_vm(issued - mark[k]);
        // per mask row: (row bits, set bits in the LT's earlier rows)
        const uint32_t mv = maskv[k];
        const uint32_t cnt = (uint32_t)__builtin_popcount(mv);
        uint32_t incl = cnt;
#pragma unroll
        for (int d = 1; d < 8; d <<= 1) {
            const uint32_t t = (uint32_t)__shfl_up((int)incl, d, 8);
            incl += (lane & 7) >= d ? t : 0u;
        }
        *(__attribute__((address_space(3))) uint64_t *)(uintptr_t)(meta_addr + 8u * (uint32_t)lane) =
                ((uint64_t)(incl - cnt) << 32) | mv;
        // B operands of the chunk's LTs
        bt_v4i xb[IE_CHUNK][NCH];
#pragma unroll
        for (int nch = 0; nch < NCH; ++nch)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bt_v4i v = ie_transpose(xg[k][nch][j]);
                xb[2 * j][nch] = bt_b_operand((uint32_t)v.x, (uint32_t)v.y);
                xb[2 * j + 1][nch] = bt_b_operand((uint32_t)v.z, (uint32_t)v.w);
            }
        const uint32_t slot_addr = slot_addr0 + (uint32_t)k * IE_SLOT_BYTES;
        const uint32_t org = g0s[k] << 5;                 // nibble index of the slot's first byte
        const uint32_t below = kg == 0 ? 0u : ((1u << (8 * kg)) - 1u);
#pragma unroll
        for (int lt = 0; lt < IE_CHUNK; ++lt) {
            if (lt >= n_lt) break;
            const uint32_t ot = (uint32_t)__builtin_amdgcn_readlane((int)offv[k], lt);
            const uint32_t ot1 = (uint32_t)__builtin_amdgcn_readlane((int)offv[k], lt + 1);
            const uint32_t P = (ot1 - ot) >> 2;
            const uint32_t rlo = (uint32_t)__builtin_amdgcn_readlane((int)rpv[k], 2 * lt);
            const uint32_t rhi = (uint32_t)__builtin_amdgcn_readlane((int)rpv[k], 2 * lt + 1);
            const uint32_t p = ((R < 8 ? rlo : rhi) >> (4 * (R & 7))) & 15u;
            const uint32_t a = p >> 3, gi = p & 7u;
            const uint2 rb = bt_lds_pair(meta_addr + 8u * (8u * (uint32_t)lt + gi));
            const uint32_t byte = __builtin_amdgcn_ubfe(rb.x, 8u * (uint32_t)kg, 8u);
            const uint32_t rank = (uint32_t)__builtin_popcount(rb.x & below) + rb.y;
            const uint2 sel = bt_lds_pair(lut_base + byte * (8u * BT_LUT_COPIES));
            const uint32_t pos0 = (ot - org) + 2u * a * P + rank;
            const uint32_t w0 = ie_window(slot_addr, pos0);
            const uint32_t w1 = ie_window(slot_addr, pos0 + P);
            uint32_t A0, A1, A2, A3;
            ie_place(w0, sel, A0, A1);
            ie_place(w1, sel, A2, A3);
            const bt_v4i av = {(int)A0, (int)A1, (int)A2, (int)A3};
#pragma unroll
            for (int nch = 0; nch < NCH; ++nch)
                acc[nch] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, xb[lt][nch], acc[nch], 0, 0, 0);
        }
        // the slot and the tables are rewritten by the next issue into them
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        if (ci == nck - 1) {
            // a band is done: its partial moves to the band's registers (a
            // select per register keeps the array statically indexed); the
            // LDS adds wait for the end, where no DMA is left in flight
#pragma unroll
            for (int b = 0; b < IE_MAXB; ++b)
#pragma unroll
                for (int nch = 0; nch < NCH; ++nch)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accb[b][nch][i] = b == bi ? acc[nch][i] : accb[b][nch][i];
#pragma unroll
            for (int nch = 0; nch < NCH; ++nch) acc[nch] = bt_v4i{0, 0, 0, 0};
        }
    };

    if (S > 0) {
        bt_wait_vm(0);                                   // chunk boundaries
        issue(0, 0);
        issue(1, 1);
        for (int s = 0; s < S; s += 2) {
            process(s, 0);
            issue(s + 2, 0);
            if (s + 1 < S) process(s + 1, 1);
            issue(s + 3, 1);
        }
        bt_wait_vm(0);
#pragma unroll
        for (int b = 0; b < IE_MAXB; ++b) {
            if (b >= nb) break;
#pragma unroll
            for (int nch = 0; nch < NCH; ++nch) {
                int32_t *sp = sums + (b * 32 + R + 16 * nch) * 16 + 4 * kg;
#pragma unroll
                for (int i = 0; i < 4; ++i) atomicAdd(&sp[i], accb[b][nch][i] >> 8);
            }
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < nb * 16 * N; o += blockDim.x) {
        const int bi = o / (16 * N), r2 = o - bi * 16 * N;
        const int n = r2 >> 4, row = r2 & 15;
        const int m = (b0 + bi) * 16 + row;
        if (m < M) Y[(int64_t)n * M + m] = sums[(bi * 32 + n) * 16 + row];
    }
}

__global__ void k_ie_zero(int32_t *__restrict__ Y, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        Y[i] = 0;
}

struct IePlan {
    int nch = 1;
    bool xu = false;
    int grid = 0, bq = 0, br = 0;
    size_t lds = IE_LDS_BYTES;
};

static bool ie_plan(int64_t M, int64_t K, int64_t N, IePlan *p) {
    if (M < 1 || K < 1 || K > IE_MAX_K || N < 1 || N > 32) return false;
    const int64_t bands = (M + 15) / 16;
    int64_t grid = std::min<int64_t>(bands, BT_CUS);
    grid = std::max<int64_t>(grid, (bands + IE_MAXB - 1) / IE_MAXB);
    if (grid > INT32_MAX) return false;
    p->grid = (int)grid;
    p->bq = (int)(bands / grid);
    p->br = (int)(bands % grid);
    p->nch = N > 16 ? 2 : 1;
    p->xu = (K % 8) != 0;
    p->lds = IE_LDS_BYTES;
    return true;
}

template <int NCH, bool XU>
static void launch_ie_t(const IePlan &p, const uint32_t *offsets, const uint64_t *ubitmaps, const uint64_t *rowpos,
                        const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                        int32_t *Y, hipStream_t stream) {
    (void)hipFuncSetAttribute((const void *)k_ie_w4a4<NCH, XU>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)p.lds);
    hipLaunchKernelGGL((k_ie_w4a4<NCH, XU>), dim3(p.grid), dim3(IE_WAVES * 64), p.lds, stream, offsets, ubitmaps,
                       rowpos, payload, payload_bytes, M, K, p.bq, p.br, X, N, Y);
}

static void launch_ie_w4a4(const IePlan &p, const uint32_t *offsets, const uint64_t *ubitmaps,
                           const uint64_t *rowpos, const uint8_t *payload, uint32_t payload_bytes, int M, int K,
                           const uint8_t *X, int N, int32_t *Y, hipStream_t stream) {
    if (p.nch == 1) {
        if (p.xu) launch_ie_t<1, true>(p, offsets, ubitmaps, rowpos, payload, payload_bytes, M, K, X, N, Y, stream);
        else launch_ie_t<1, false>(p, offsets, ubitmaps, rowpos, payload, payload_bytes, M, K, X, N, Y, stream);
    } else {
        if (p.xu) launch_ie_t<2, true>(p, offsets, ubitmaps, rowpos, payload, payload_bytes, M, K, X, N, Y, stream);
        else launch_ie_t<2, false>(p, offsets, ubitmaps, rowpos, payload, payload_bytes, M, K, X, N, Y, stream);
    }
}
