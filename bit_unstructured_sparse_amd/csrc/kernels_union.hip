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
// the wavefront's slots (IE_NSLOT at N <= 16, two above), and their X columns
// as 16-byte granules, all issued as many steps ahead as there are slots
// after the first. Slots, tables and X are private to the wavefront, so
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
#define IE_NSLOT 3                    // payload slots per wavefront: steps in flight
#define IE_LUT_COPIES 8               // selector-table copies (lane l reads copy l % 8)
#define IE_LUT_BYTES (2048 * IE_LUT_COPIES)
#define IE_SUMS_BYTES (IE_MAXB * 32 * 16 * 4)
#define IE_LDS_BYTES (IE_SUMS_BYTES + IE_LUT_BYTES + IE_WAVES * IE_META_BYTES + IE_WAVES * IE_NSLOT * IE_SLOT_BYTES)
#define IE_MAX_K BSP_UNION_MAX_K
#define IE_OOR 0xFFFFFFF0u            // a buffer offset past every range: reads zeros

// Eight payload-window reads (two dwords each, at LDS byte addresses a0[i]
// and a1[i], i < 4), completed before the block ends: the outputs are
// written when the block's own wait returns, never later.
__device__ __forceinline__ void ie_read_windows(const uint32_t *a0, const uint32_t *a1, uint64_t *d0,
                                                uint64_t *d1) {
    asm volatile(
            "ds_read2_b32 %0, %8 offset1:1\n\t"
            "ds_read2_b32 %1, %9 offset1:1\n\t"
            "ds_read2_b32 %2, %10 offset1:1\n\t"
            "ds_read2_b32 %3, %11 offset1:1\n\t"
            "ds_read2_b32 %4, %12 offset1:1\n\t"
            "ds_read2_b32 %5, %13 offset1:1\n\t"
            "ds_read2_b32 %6, %14 offset1:1\n\t"
            "ds_read2_b32 %7, %15 offset1:1\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(d0[0]), "=&v"(d1[0]), "=&v"(d0[1]), "=&v"(d1[1]), "=&v"(d0[2]), "=&v"(d1[2]), "=&v"(d0[3]),
              "=&v"(d1[3])
            : "v"(a0[0]), "v"(a1[0]), "v"(a0[1]), "v"(a1[1]), "v"(a0[2]), "v"(a1[2]), "v"(a0[3]), "v"(a1[3])
            : "memory");
}

// Four LDS integer adds at byte address a (a, a + 4, a + 8, a + 12). Issued
// as LDS instructions the compiler would first wait for every LDS DMA in
// flight; they have no outputs, and the kernel waits for them (lgkmcnt)
// before its final barrier.
__device__ __forceinline__ void ie_add4(uint32_t a, bt_v4i v) {
    asm volatile(
            "ds_add_u32 %0, %1\n\t"
            "ds_add_u32 %0, %2 offset:4\n\t"
            "ds_add_u32 %0, %3 offset:8\n\t"
            "ds_add_u32 %0, %4 offset:12"
            :
            : "v"(a), "v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w)
            : "memory");
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
    uint8_t *meta8 = lut8 + IE_LUT_BYTES + wave * IE_META_BYTES;
    uint8_t *slot8 = lut8 + IE_LUT_BYTES + IE_WAVES * IE_META_BYTES + wave * IE_NSLOT * IE_SLOT_BYTES;
    const uint32_t lut_base = bt_lds_addr(lut8) + (uint32_t)(lane % IE_LUT_COPIES) * 8u;
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
    for (int e = threadIdx.x; e < 256 * IE_LUT_COPIES; e += blockDim.x) {
        const uint2 v = bt_lut_entry((uint32_t)e / IE_LUT_COPIES);
        *reinterpret_cast<uint2 *>(lut8 + (size_t)e * 8) = v;
    }
    __syncthreads();

    // slots in use: all IE_NSLOT at N <= 16; two at N > 16, whose X granules
    // take twice the registers
    constexpr int NS = NCH == 1 ? IE_NSLOT : 2;
    uint32_t maskv[NS], rpv[NS], offv[NS], g0s[NS], mark[NS] = {};
    bt_v4i xg[NS][NCH][4];
    uint32_t xe[NS][NCH][4];

    // Issue the loads of step s into slot k. A step past the last one issues
    // the same instructions with every offset out of range (they read zeros
    // and move no data): the count per step is then fixed, so every wait
    // below is exact.
    auto issue = [&](int s, int k) {
        const bool live = s < S;
        const int ci = live ? s / nb : 0, bi = live ? s - ci * nb : 0;
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
                // K % 8 != 0: rows are not dword aligned; the 20 bytes from the
                // dword boundary below are loaded now and shifted into place
                // when used, so nothing waits for them here
                const uint32_t a = XU ? (off & ~3u) : off;
                xg[k][nch][j] = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, a, 0, 0));
                if constexpr (XU) xe[k][nch][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(xrs, a + 16u, 0, 0);
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

    bt_v4i xb[IE_CHUNK][NCH];              // B operands of the current chunk

    auto process = [&](int s, int k) {
        const int ci = s / nb, bi = s - ci * nb;
        const int cc0 = c0 + IE_CHUNK * ci;
        const int n_lt = min(IE_CHUNK, c1 - cc0);
        bt_wait_vm(issued - mark[k]);
        // per mask row: (row bits, set bits in the LT's earlier rows); the
        // prefix runs over each LT's 8 rows (8 lanes)
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
        const uint32_t slot_addr = slot_addr0 + (uint32_t)k * IE_SLOT_BYTES;
        const uint32_t org = g0s[k] << 5;                 // nibble index of the slot's first byte
        const uint32_t below = kg == 0 ? 0u : ((1u << (8 * kg)) - 1u);
        // The step's LTs go through three phases, each over all IE_CHUNK of
        // them with no branch, so each phase's LDS reads are in flight
        // together: (1) the lane's mask row, (2) its selector pair and two
        // payload windows, (3) decode and MFMA. An LT past the chunk's end has
        // an empty mask (its mask dwords read as zeros): its selectors give
        // zeros and its windows are read at the slot's start.
        uint2 rb[IE_CHUNK];
        uint32_t aP2[IE_CHUNK], Pl[IE_CHUNK], base[IE_CHUNK];
#pragma unroll
        for (int lt = 0; lt < IE_CHUNK; ++lt) {
            const bool in = lt < n_lt;
            const uint32_t ot_l = (uint32_t)__builtin_amdgcn_readlane((int)offv[k], lt);
            const uint32_t ot1_l = (uint32_t)__builtin_amdgcn_readlane((int)offv[k], lt + 1);
            const uint32_t ot = in ? ot_l : org, ot1 = in ? ot1_l : org;
            Pl[lt] = (ot1 - ot) >> 2;
            base[lt] = ot - org;
            const uint32_t rlo = (uint32_t)__builtin_amdgcn_readlane((int)rpv[k], 2 * lt);
            const uint32_t rhi = (uint32_t)__builtin_amdgcn_readlane((int)rpv[k], 2 * lt + 1);
            const uint32_t p = (uint32_t)((((uint64_t)rhi << 32) | rlo) >> (4 * R)) & 15u;
            aP2[lt] = (p >> 3) ? 2u * Pl[lt] : 0u;       // stream 2a starts 2 a P values in
            rb[lt] = bt_lds_pair(meta_addr + 8u * (8u * (uint32_t)lt + (p & 7u)));
        }
        uint2 sel[IE_CHUNK];
        uint64_t d0[IE_CHUNK], d1[IE_CHUNK];
        uint32_t sh0[IE_CHUNK], sh1[IE_CHUNK], wa0[IE_CHUNK], wa1[IE_CHUNK];
#pragma unroll
        for (int lt = 0; lt < IE_CHUNK; ++lt) {
            const uint32_t byte = __builtin_amdgcn_ubfe(rb[lt].x, 8u * (uint32_t)kg, 8u);
            const uint32_t rank = (uint32_t)__builtin_popcount(rb[lt].x & below) + rb[lt].y;
            sel[lt] = bt_lds_pair(lut_base + byte * (8u * IE_LUT_COPIES));
            const uint32_t pos0 = base[lt] + aP2[lt] + rank;
            const uint32_t pos1 = pos0 + Pl[lt];
            wa0[lt] = slot_addr + ((pos0 >> 3) << 2);
            wa1[lt] = slot_addr + ((pos1 >> 3) << 2);
            // the funnel shift reads the low 5 bits of its amount: 4 (pos & 7)
            sh0[lt] = pos0 << 2;
            sh1[lt] = pos1 << 2;
        }
        // The window reads of the slot. Written out as LDS instructions the
        // compiler would precede them with a wait for every LDS DMA still in
        // flight (the later steps' too): it cannot tell the slots apart. The
        // step's own DMAs are complete (the counted wait above), so the reads
        // are issued here, four LTs per block, and each block waits for its
        // own reads before it ends.
        ie_read_windows(&wa0[0], &wa1[0], &d0[0], &d1[0]);
        ie_read_windows(&wa0[4], &wa1[4], &d0[4], &d1[4]);
        // A chunk's first step (band 0) builds the B operands of its LTs from
        // the X granules that came with it; the chunk's other bands reuse them
        if (bi == 0) {
#pragma unroll
            for (int j = 0; j < IE_CHUNK / 2; ++j)
#pragma unroll
                for (int nch = 0; nch < NCH; ++nch) {
                    bt_v4i g = xg[k][nch][j];
                    if constexpr (XU) {
                        const uint32_t sh = ((uint32_t)(R + 16 * nch) * xs) & 3u;
                        const uint32_t e = xe[k][nch][j];
                        g = bt_v4i{(int)__builtin_amdgcn_alignbyte((uint32_t)g.y, (uint32_t)g.x, sh),
                                   (int)__builtin_amdgcn_alignbyte((uint32_t)g.z, (uint32_t)g.y, sh),
                                   (int)__builtin_amdgcn_alignbyte((uint32_t)g.w, (uint32_t)g.z, sh),
                                   (int)__builtin_amdgcn_alignbyte(e, (uint32_t)g.w, sh)};
                    }
                    const bt_v4i t = ie_transpose(g);
                    xb[2 * j][nch] = bt_b_operand((uint32_t)t.x, (uint32_t)t.y);
                    xb[2 * j + 1][nch] = bt_b_operand((uint32_t)t.z, (uint32_t)t.w);
                }
        }
        bt_v4i acc[NCH];
#pragma unroll
        for (int lt = 0; lt < IE_CHUNK; ++lt) {
            uint32_t A0, A1, A2, A3;
            ie_place(__builtin_amdgcn_alignbit((uint32_t)(d0[lt] >> 32), (uint32_t)d0[lt], sh0[lt]), sel[lt], A0, A1);
            ie_place(__builtin_amdgcn_alignbit((uint32_t)(d1[lt] >> 32), (uint32_t)d1[lt], sh1[lt]), sel[lt], A2, A3);
            const bt_v4i av = {(int)A0, (int)A1, (int)A2, (int)A3};
#pragma unroll
            for (int nch = 0; nch < NCH; ++nch)
                acc[nch] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, xb[lt][nch], lt == 0 ? bt_v4i{0, 0, 0, 0} : acc[nch],
                                                                 0, 0, 0);
        }
        // the step's partial (exact after >> 8) joins its band's sums in LDS
#pragma unroll
        for (int nch = 0; nch < NCH; ++nch)
            ie_add4(bt_lds_addr(sums + (bi * 32 + R + 16 * nch) * 16 + 4 * kg), acc[nch] >> 8);
        // the slot and the tables are rewritten by the next issue into them
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
    };

    if (S > 0) {
        bt_wait_vm(0);                                   // chunk boundaries
#pragma unroll
        for (int k = 0; k < NS; ++k) issue(k, k);
        for (int s = 0; s < S; s += NS) {
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                if (k == 0 || s + k < S) process(s + k, k);
                issue(s + k + NS, k);
            }
        }
        bt_wait_vm(0);
    }
    // the LDS adds above were issued outside the compiler's view: wait for them
    __builtin_amdgcn_s_waitcnt(0xC07F);
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
