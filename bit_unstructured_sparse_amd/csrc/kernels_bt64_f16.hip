// kernels_bt64_f16.hip -- block-staged bitmap decode + fp16 MFMA contraction
// for the fp16 SpMM (u16 payload, fp16 X, fp32 accumulation, fp16 Y) on
// gfx950. Included after kernels_bt64.hip, whose helpers it uses.
//
// The stream is the same BT64 format with 2-byte values (the column-bitmap
// kernel of SPDP, Sec. 4.2, stores FP16 values the same way: one bit per
// position, values packed in position order). The skeleton is the int4
// kernel's: 16-row blocks, a workgroup per CU owning a contiguous run of
// blocks, each block's payload staged into LDS by DMA from its two boundary
// offsets, lane starts from bitmap popcounts, one barrier per block.
//
// Work split. One tile per lane: lane l = r + 16 q of wavefront w owns row r
// and tile 4 w + q, so a block of T <= 64 tiles takes ceil(T / 4) <= 16
// wavefronts. A lane keeps its tile's X (64 halves per column) in VGPRs.
//
// Decode of 4 positions (one nibble m of the word). The 4 values they can
// need start at the lane's element p: the two dwords holding halves p .. p+3
// come from three staged dwords and one funnel shift by 16 * (p & 1). Two
// v_perm_b32 then place the nibble's nonzeros (in rank order in the window)
// at their positions and zero the rest; the selector pair comes from a
// 16-entry table indexed by m. Two nibbles make the 8 halves a lane feeds to
// one v_mfma_f32_16x16x32_f16; MFMA j of a tile contracts positions
// 8j .. 8j+7 of every lane's tile with the matching X slice (the K order
// inside one MFMA is free as long as A and B use the same one).
//
// Sums. Each wavefront stores its fp32 partial of a block to its own LDS
// slice; after the next barrier the slices are added in wavefront order and
// rounded once to fp16 (round to nearest even), so a result does not depend
// on timing.

#define BF_ROWS 16
#define BF_MAX_WAVES 16
#define BF_NBLK 4                        // blocks per workgroup, at most
#define BF_LDS_MAX (160 * 1024)
#define BF_CUS 256

typedef _Float16 bf_h8 __attribute__((ext_vector_type(8)));
typedef float bf_f4 __attribute__((ext_vector_type(4)));

// Selector table: entry m (a 4-bit group of the word) is the v_perm_b32
// selector pair for output dwords {positions 0,1} and {positions 2,3}; the
// perm's sources are S0 = window halves 2,3 (selector bytes 4..7) and
// S1 = window halves 0,1 (0..3), and selector 0x0C yields a zero byte. Built
// in LDS by the kernel itself.

// Payload range of a block in 16-byte granules: [g0, g0 + n) covers halves
// [eA, eB) plus one granule for the windows that read past the last value.
__device__ __forceinline__ BtRange bf_range(uint32_t eA, uint32_t eB) {
    const uint32_t g0 = eA >> 3;
    const uint32_t g1 = (eB >= eA ? (eB + 7u) >> 3 : g0) + 1u;
    return BtRange{g0, g1 - g0};
}

// Window source: the staged stream in LDS; p counts halves from half the
// buffer's LDS address (a multiple of 16), so dword p >> 1 of the stream sits
// at byte address (p << 1) & ~3 and p & 1 is the half inside it.
struct BfWinLds {
    __device__ __forceinline__ uint2 operator()(uint32_t p) const {
        const bt_lds_u32 *q = (const bt_lds_u32 *)(uintptr_t)((p << 1) & ~3u);
        const uint32_t d0 = q[0], d1 = q[1], d2 = q[2];
        const uint32_t s = p << 4;   // funnel shift by 16 * (p & 1)
        return uint2{__builtin_amdgcn_alignbit(d1, d0, s), __builtin_amdgcn_alignbit(d2, d1, s)};
    }
};

// Window source: global memory (p counts halves from payload dword d0).
struct BfWinGlobal {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t d0;
    __device__ __forceinline__ uint2 operator()(uint32_t p) const {
        const uint32_t off = (d0 + (p >> 1)) * 4u;
        const uint32_t a = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
        const uint32_t b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off + 4u, 0, 0);
        const uint32_t c = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off + 8u, 0, 0);
        const uint32_t s = p << 4;
        return uint2{__builtin_amdgcn_alignbit(b, a, s), __builtin_amdgcn_alignbit(c, b, s)};
    }
};

// The same for a staged stream, software-pipelined: the stream positions of
// all 16 groups first, then each byte's window and selector reads are issued
// one byte ahead of the placement that uses them (scheduling fences keep the
// compiler from sinking the reads back to their use; one byte of lookahead
// keeps about 8 LDS reads in flight at 20 more registers).
template <int NB>
__device__ __forceinline__ void bf_contract_lds_ahead(uint64_t word, uint32_t p, uint32_t lut,
                                                      const bf_h8 (&xb)[NB][8], bf_f4 (&acc)[NB]) {
    uint32_t pp[16], mm[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        mm[k] = (uint32_t)(word >> (4 * k)) & 15u;
        pp[k] = p;
        p = (uint32_t)__builtin_popcount(mm[k]) + p;
    }
    uint32_t d0[16], d1[16], d2[16];
    uint2 ss[16];
    auto rd = [&](int j) -> void {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * j + h;
            ss[k] = bt_lds_pair(lut + mm[k] * 8u);
            const bt_lds_u32 *q = (const bt_lds_u32 *)(uintptr_t)((pp[k] << 1) & ~3u);
            d0[k] = q[0];
            d1[k] = q[1];
            d2[k] = q[2];
        }
    };
    rd(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j + 1 < 8) rd(j + 1);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t A[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * j + h;
            const uint32_t s = pp[k] << 4;   // funnel shift by 16 * (p & 1)
            const uint32_t wx = __builtin_amdgcn_alignbit(d1[k], d0[k], s);
            const uint32_t wy = __builtin_amdgcn_alignbit(d2[k], d1[k], s);
            A[2 * h] = __builtin_amdgcn_perm(wy, wx, ss[k].x);
            A[2 * h + 1] = __builtin_amdgcn_perm(wy, wx, ss[k].y);
        }
        const bf_h8 a = __builtin_bit_cast(bf_h8, bt_v4i{(int)A[0], (int)A[1], (int)A[2], (int)A[3]});
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, xb[nb][j], acc[nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// X granules loaded with lane group q holding granules 4 i + q (i = 0..7) of
// its wavefront's four tiles -> each lane's own tile q, granule j in xb[.][j].
// Element E[q][s] = (xg[2s], xg[2s+1]) = granules 8s + q and 8s + 4 + q; the
// 4 x 4 transpose over (q, s) leaves E[s][q] in slot s of group q, i.e.
// granules 8q + s and 8q + 4 + s: j = s and j = 4 + s of tile q. Two stages
// of swaps between lane groups: q ^ 2 (32-lane swap: the upper half of its
// first operand with the lower half of its second) on slots s and s + 2, then
// q ^ 1 (16-lane swap: the odd rows of the first with the even rows of the
// second) on slots 2u and 2u + 1. Every lane must be active.
template <int NB>
__device__ __forceinline__ void bf_x_transpose(bt_v4i (&xg)[NB][8], bf_h8 (&xb)[NB][8]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const auto w = __builtin_amdgcn_permlane32_swap((unsigned)xg[nb][2 * s + e][d],
                                                                    (unsigned)xg[nb][2 * (s + 2) + e][d], false, false);
                    xg[nb][2 * s + e][d] = (int)w[0];
                    xg[nb][2 * (s + 2) + e][d] = (int)w[1];
                }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const auto w = __builtin_amdgcn_permlane16_swap((unsigned)xg[nb][2 * (2 * u) + e][d],
                                                                    (unsigned)xg[nb][2 * (2 * u + 1) + e][d], false, false);
                    xg[nb][2 * (2 * u) + e][d] = (int)w[0];
                    xg[nb][2 * (2 * u + 1) + e][d] = (int)w[1];
                }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xb[nb][s] = __builtin_bit_cast(bf_h8, xg[nb][2 * s]);
            xb[nb][4 + s] = __builtin_bit_cast(bf_h8, xg[nb][2 * s + 1]);
        }
    }
}

// Decode + contract one tile: 8 MFMAs of 8 positions each.
template <int NB, class Win>
__device__ __forceinline__ void bf_contract(uint64_t word, uint32_t p, const Win &win, uint32_t lut,
                                            const bf_h8 (&xb)[NB][8], bf_f4 (&acc)[NB]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t A[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t m = (uint32_t)(word >> (8 * j + 4 * h)) & 15u;
            const uint2 sel = bt_lds_pair(lut + m * 8u);
            const uint2 w = win(p);
            A[2 * h] = __builtin_amdgcn_perm(w.y, w.x, sel.x);
            A[2 * h + 1] = __builtin_amdgcn_perm(w.y, w.x, sel.y);
            p = (uint32_t)__builtin_popcount(m) + p;
        }
        const bf_h8 a = __builtin_bit_cast(bf_h8, bt_v4i{(int)A[0], (int)A[1], (int)A[2], (int)A[3]});
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, xb[nb][j], acc[nb], 0, 0, 0);
    }
}

// LDS layout (bytes): [selector table 128][row totals 2 x 16 x 16 ints]
//   [partials P x nwaves x NB x 256 floats][nbuf staging buffers of stage_bytes]
// with P = psets partial sets: 2 (block i adds into set i % 2 while set
// (i - 1) % 2 is summed into Y), or 1 (one block per workgroup; or several,
// block i's partials written after a barrier that follows the sum of block
// i - 1), as the plan fits them.
// Workgroup g owns blocks [g*bq + min(g, br), ...): bq or bq + 1 of them.
template <int NB>
__global__ __launch_bounds__(1024) void k_bt64_f16(
        const uint64_t *__restrict__ bitmaps, const uint32_t *__restrict__ offsets,
        const uint16_t *__restrict__ payload, uint32_t payload_bytes, int M, int K,
        const uint16_t *__restrict__ X, int N, uint16_t *__restrict__ Y, uint32_t stage_bytes, uint32_t nbuf,
        int bq, int br, int psets) {
    extern __shared__ __attribute__((aligned(16))) uint8_t bf_smem[];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int T = (K + 63) >> 6;
    const int gid = (int)blockIdx.x;
    const int b_begin = gid * bq + min(gid, br);
    const int nblk = bq + (gid < br ? 1 : 0);           // 1 .. BF_NBLK
    const int t = wave * 4 + q;                          // this lane's tile

    uint32_t *lut_lds = reinterpret_cast<uint32_t *>(bf_smem);
    int32_t *wt = reinterpret_cast<int32_t *>(bf_smem + 128);                           // [2][16][16]
    float *part = reinterpret_cast<float *>(wt + 2 * BF_ROWS * BF_MAX_WAVES);            // [P][nwaves][NB*256]
    uint8_t *stage = reinterpret_cast<uint8_t *>(part + psets * nwaves * NB * 256);
    const uint32_t lut = bt_lds_addr(lut_lds);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(payload, payload_bytes);

    // every kernel argument into SGPRs in the first batch of argument loads
    // (one loaded after the offsets below would wait for those too)
    asm volatile("" ::"s"(bitmaps), "s"(payload), "s"(X), "s"(Y), "s"(N), "s"(stage_bytes), "s"(nbuf),
                 "s"(payload_bytes));

    // (1) block boundaries (wave-uniform scalar loads)
    uint32_t eb[BF_NBLK + 1];
#pragma unroll
    for (int i = 0; i <= BF_NBLK; ++i) {
        const int b = b_begin + (i < nblk ? i : nblk);
        eb[i] = offsets[(int64_t)min(b * BF_ROWS, M) * T];
    }
    // keep these loads issued here, ahead of the vector loads (the compiler
    // would otherwise sink them to their first use, behind every wait)
    asm volatile("" ::: "memory");

    // (2) loads that need no offsets first (waiting for them then never
    // waits for a payload DMA): the selector table, this lane's X, every
    // block's bitmap word; after the offsets land, the payload DMA of the
    // first nbuf blocks (16-byte granules in stream order into staging buffer
    // i % nbuf). A block that does not fit is not staged: it reads its
    // windows from global memory.
    uint32_t vm_issued = 0, vm_mark[BF_NBLK];
    // this lane's X: column r + 16 nb, positions 64 t .. 64 t + 63, as the
    // B operands of the tile's 8 MFMAs (column n >= N or tile >= T: zeros).
    // The wavefront's four tiles are 512 contiguous bytes of each X row. Load
    // i gives lane group q the 16-byte granule 4 i + q of them, so one load
    // covers 64-byte runs of 16 rows instead of one line per lane (the line
    // requests, not the bytes, bound this prologue); a transpose across the
    // lane groups (bf_x_transpose, in block 0) then hands each lane its own
    // tile's granules.
    bt_v4i xg[NB][8];
    {
        const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(X, (uint32_t)N * (uint32_t)K * 2u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = r + 16 * nb;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t gi = 4u * (uint32_t)i + (uint32_t)q;       // granule of the wavefront's 512 bytes
                const uint32_t tt = (uint32_t)(wave * 4) + (gi >> 3);       // its tile
                // positions past K read as zeros too: a finite weight of 0 times
                // a non-finite X from the next row would give NaN
                const uint32_t k0 = tt * 64u + 8u * (gi & 7u);
                const uint32_t off = (n < N && tt < (uint32_t)T && k0 < (uint32_t)K)
                                             ? ((uint32_t)n * (uint32_t)K + k0) * 2u : 0xFFFFFFF0u;
                xg[nb][i] = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
            }
        }
        vm_issued += NB * 8;
    }
    bf_h8 xb[NB][8];
    const int m_first = b_begin * BF_ROWS;
    const int wg_rows = min(nblk * BF_ROWS, M - m_first);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(bitmaps + (int64_t)m_first * T, (uint32_t)wg_rows * (uint32_t)T * 8u);
    uint64_t words[BF_NBLK];
#pragma unroll
    for (int i = 0; i < BF_NBLK; ++i) {
        // every slot is loaded (past nblk: zeros), so the loads in flight can be counted
        const int rr = i * BF_ROWS + r;
        const uint32_t off = (rr < wg_rows && t < T) ? ((uint32_t)rr * (uint32_t)T + (uint32_t)t) * 8u : 0xFFFFFFF0u;
        words[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off, 0, 0));
        ++vm_issued;
    }
    // the 16-entry selector table, computed in registers (lane m: entry m)
    if (threadIdx.x < 16) {
        const uint32_t m = threadIdx.x;
        uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu};
#pragma unroll
        for (int pos = 0; pos < 4; ++pos) {
            const uint32_t rank = (uint32_t)__builtin_popcount(m & ((1u << pos) - 1u));
            const uint32_t v = (2u * rank) | ((2u * rank + 1u) << 8);   // bytes of half `rank`
            const uint32_t sh = 16u * (uint32_t)(pos & 1);
            const uint32_t upd = (sel[pos >> 1] & ~(0xFFFFu << sh)) | (v << sh);
            sel[pos >> 1] = ((m >> pos) & 1u) ? upd : sel[pos >> 1];
        }
        lut_lds[2 * m] = sel[0];
        lut_lds[2 * m + 1] = sel[1];
    }

    auto fits = [&](int i) -> bool { return bf_range(eb[i], eb[i + 1]).n * 16u <= stage_bytes; };
    auto issue_block = [&](int i) -> void {
        if (fits(i)) {
            const BtRange g = bf_range(eb[i], eb[i + 1]);
            uint8_t *buf = stage + (uint32_t)(i % (int)nbuf) * stage_bytes;
            const uint32_t n_ins = (g.n + 63u) >> 6;
            for (uint32_t j = (uint32_t)wave; j < n_ins; j += (uint32_t)nwaves) {
                const uint32_t u = j * 64u + (uint32_t)lane;
                if (u < g.n)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(buf + j * 1024u), 16,
                                                             (g.g0 + u) * 16u, 0, 0, BT_NT);
                ++vm_issued;
            }
        }
        vm_mark[i] = vm_issued;
    };
#pragma unroll
    for (int i = 0; i < BF_NBLK; ++i) {
        vm_mark[i] = vm_issued;   // the words; staging the block raises it
        if (i < nblk && i < (int)nbuf) issue_block(i);
    }

    // (4) blocks in order, one barrier each (as in the int4 kernel): before
    // the barrier of block i each wavefront posts its row totals; after it,
    // lane starts are known, block i-1's partials are complete and its
    // staging buffer is free. Partials alternate between two buffers.
    auto write_y = [&](int i) -> void {
        const int m0 = (b_begin + i) * BF_ROWS;
        const int rows = min(BF_ROWS, M - m0);
        const float *pb = part + (psets == 2 ? (i & 1) : 0) * nwaves * NB * 256;
        // D layout of the 16x16 MFMAs: lane l, register k -> row 4*(l/16)+k, column l%16
        for (int o = threadIdx.x; o < NB * 256; o += blockDim.x) {
            const int nb = o >> 8, col = (o >> 4) & 15, rl = o & 15;
            const int ln = (rl >> 2) * 16 + col, k = rl & 3;
            const int n = col + 16 * nb;
            if (n < N && rl < rows) {
                float s = 0.f;
                for (int w = 0; w < nwaves; ++w) s += pb[(w * NB + nb) * 256 + k * 64 + ln];
                Y[(int64_t)n * M + m0 + rl] = __builtin_bit_cast(uint16_t, (_Float16)s);
            }
        }
    };
#pragma unroll
    for (int i = 0; i < BF_NBLK; ++i) {
        if (i >= nblk) break;
        const bool in_lds = fits(i);
        const BtRange g = bf_range(eb[i], eb[i + 1]);
        const int rows = min(BF_ROWS, M - (b_begin + i) * BF_ROWS);

        // this lane's tile popcount, inclusive prefix over q
        const uint32_t seg = (uint32_t)__builtin_popcountll(words[i]);
        uint32_t incl = seg;
        {
            const uint32_t u16 = (uint32_t)__shfl_up((int)incl, 16, 64);
            incl += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)incl, 32, 64);
            incl += q >= 2 ? u32 : 0u;
        }
        int32_t *wti = wt + (i & 1) * BF_ROWS * BF_MAX_WAVES;
        if (q == 3) wti[r * BF_MAX_WAVES + wave] = (int32_t)incl;   // this wavefront's total for row r

        bt_wait_vm(vm_issued - vm_mark[i]);
        __syncthreads();
        if (i > 0) {
            write_y(i - 1);
            if (i - 1 + (int)nbuf < nblk) issue_block(i - 1 + (int)nbuf);
        }

        // lane start: rows before r, wavefronts before this one, lane groups before q
        uint32_t pstart;
        {
            uint32_t row_total = 0, before_w = 0;
            const bt_lds_v4i *tv = (const bt_lds_v4i *)(uintptr_t)bt_lds_addr(wti + r * BF_MAX_WAVES);
#pragma unroll
            for (int v = 0; v < BF_MAX_WAVES / 4; ++v) {
                const bt_v4i t4 = tv[v];
                const uint32_t tw[4] = {(uint32_t)t4.x, (uint32_t)t4.y, (uint32_t)t4.z, (uint32_t)t4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int w = 4 * v + e;
                    const uint32_t val = w < nwaves ? tw[e] : 0u;
                    row_total += val;
                    if (w < wave) before_w += val;
                }
            }
            uint32_t s = row_total;
            s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0x111, 0xF, 0xF, true);   // row_shr:1
            s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0x112, 0xF, 0xF, true);   // row_shr:2
            s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0x114, 0xF, 0xF, true);   // row_shr:4
            s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, 0x118, 0xF, 0xF, true);   // row_shr:8
            // element index of the lane's first nonzero, counted from the block's first granule
            pstart = r < rows ? (eb[i] & 7u) + (s - row_total) + before_w + (incl - seg) : 0u;
        }

        if (i == 0) bf_x_transpose<NB>(xg, xb);
        bf_f4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = bf_f4{0.f, 0.f, 0.f, 0.f};
        uint32_t p = pstart;
        if (in_lds) {
            p = min(p, 2u * (4u * g.n - 3u));   // a corrupt stream stays inside the staged granules
            p += bt_lds_addr(stage + (uint32_t)(i % (int)nbuf) * stage_bytes) >> 1;
            bf_contract<NB>(words[i], p, BfWinLds{}, lut, xb, acc);
        } else {
            bf_contract<NB>(words[i], p, BfWinGlobal{prs, 4u * g.g0}, lut, xb, acc);
        }
        float *pw = part + (psets == 2 ? (i & 1) : 0) * nwaves * NB * 256 + wave * NB * 256;
        if (psets == 1 && i > 0) __syncthreads();   // block i - 1's sum has read the one set
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < 4; ++k) pw[nb * 256 + k * 64 + lane] = acc[nb][k];
    }
    __syncthreads();
    write_y(nblk - 1);
}

// ---------------------------------------------------------------------------
// Eight-row steps (N <= 8, K <= 4096). A workgroup walks its rows eight at a
// time; the payload of eight consecutive rows is one contiguous piece of the
// stream, so a step's payload can be in flight while the previous step is
// decoded, also when a workgroup owns a single 16-row block (the fp16
// configuration here: 4096 rows over 256 CUs). The 16 A rows of an MFMA hold
// the step's 8 rows twice: lanes r < 8 take row r over the first half of the
// tiles, lanes r >= 8 row r - 8 over the second half. B column n < 8 carries
// X column n over the first half, column 8 + n the same X column over the
// second half, so D[i][n] and D[8 + i][8 + n] are the two halves of row i,
// column n (the other entries mix halves and are dropped): one MFMA per 8
// positions, as in the 16-row kernel, with one accumulator. A lane's X tile is
// the same tile as its A tile.
//
// Lane starts: a lane loads the start of its half row from the offsets (one
// 4-byte load per lane and step) and adds the popcounts of the tiles before
// its own in that half row: earlier wavefronts through the row totals posted
// to LDS before the step's barrier, earlier lane groups by lane shuffles.
//
// Payload: 1 KB DMA instructions into a staging area of area_kb KB, dealt
// round robin to the wavefronts; one step in flight (step s + 1 is issued
// once step s has landed), areas used in a ring of three so that the area a
// DMA fills was last read two barriers earlier. A step larger than the area
// reads its windows from global memory.
#define BF8_NSTEP_MAX 8                  // steps per workgroup, at most (NSTEP 2, 4 or 8)
#define BF8_WAVES 8

template <int NSTEP, bool XR, bool RING = false>
__global__ __launch_bounds__(512) void k_bt8_f16(
        const uint32_t *__restrict__ offsets, int M, int K, int sq, int sr, const uint64_t *__restrict__ bitmaps,
        const uint16_t *__restrict__ X, int N, const uint16_t *__restrict__ payload, uint32_t payload_bytes,
        uint16_t *__restrict__ Y, uint32_t area_kb) {
    extern __shared__ __attribute__((aligned(16))) uint8_t bf_smem[];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int row8 = r & 7, kh = r >> 3;
    const int T = (K + 63) >> 6, T2 = (T + 1) >> 1;
    const int tw = wave * 4 + q;                 // tile inside the half row
    const int t = kh * T2 + tw;                  // this lane's tile (A and X)
    const bool tile_ok = tw < T2 && t < T;
    const int gid = (int)blockIdx.x;
    const int s_begin = gid * sq + min(gid, sr);   // first step (8-row unit) of this workgroup
    const int nstep = sq + (gid < sr ? 1 : 0);     // 1 .. NSTEP
    const int nstep_max = sq + (sr > 0 ? 1 : 0);
    asm volatile("" ::"s"(bitmaps), "s"(payload), "s"(X), "s"(Y), "s"(N), "s"(payload_bytes), "s"(area_kb));

    // LDS: selector table (128 B) | row totals [NSTEP][16][8] | partials
    // [nstep_max][nwaves][256] floats, summed into Y at the end (RING:
    // [min(nstep_max, 2)], step i in slot i % 2, summed after the next
    // step's barrier; 0.45 us slower at 2 steps, 1 us at 8 where both fit) |
    // staging [min(nstep_max, 3)][area_kb KB]
    uint32_t *lut_lds = reinterpret_cast<uint32_t *>(bf_smem);
    int32_t *wt = reinterpret_cast<int32_t *>(bf_smem + 128);
    float *part = reinterpret_cast<float *>(wt + NSTEP * BF_ROWS * BF8_WAVES);
    uint8_t *stage = reinterpret_cast<uint8_t *>(part + (RING ? min(nstep_max, 2) : nstep_max) * nwaves * 256);
    const uint32_t area = area_kb * 1024u;
    const uint32_t cap = area_kb * 64u;           // granules an area holds
    const uint32_t lut = bt_lds_addr(lut_lds);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(payload, payload_bytes);

    // step boundaries (wave-uniform scalar loads), ahead of everything
    uint32_t eb[NSTEP + 1];
#pragma unroll
    for (int i = 0; i <= NSTEP; ++i) {
        const int s = s_begin + (i < nstep ? i : nstep);
        eb[i] = offsets[(int64_t)min(s * 8, M) * T];
    }
    asm volatile("" ::: "memory");

    // every step's word and half-row start (rows past M read zeros: past the
    // end of the buffers; a tile past its half is cleared before use)
    const int m_first = s_begin * 8;
    const int wg_rows = max(0, min(nstep * 8, M - m_first));
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(bitmaps + (int64_t)m_first * T, (uint32_t)wg_rows * (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t ors = bt_rsrc(offsets + (int64_t)m_first * T, (uint32_t)wg_rows * (uint32_t)T * 4u);
    uint64_t words[NSTEP];
    uint32_t hs[NSTEP];
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        const uint32_t row = (uint32_t)(i * 8 + row8);   // inside the workgroup's range
        words[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                        brs, (row * (uint32_t)T + (uint32_t)t) * 8u, 0, 0));
        hs[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ors, (row * (uint32_t)T + (uint32_t)(kh * T2)) * 4u,
                                                               0, 0);
    }
    // the 16-entry selector table (as in the 16-row kernel)
    if (threadIdx.x < 16) {
        const uint32_t m = threadIdx.x;
        uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu};
#pragma unroll
        for (int pos = 0; pos < 4; ++pos) {
            const uint32_t rank = (uint32_t)__builtin_popcount(m & ((1u << pos) - 1u));
            const uint32_t v = (2u * rank) | ((2u * rank + 1u) << 8);
            const uint32_t sh = 16u * (uint32_t)(pos & 1);
            const uint32_t upd = (sel[pos >> 1] & ~(0xFFFFu << sh)) | (v << sh);
            sel[pos >> 1] = ((m >> pos) & 1u) ? upd : sel[pos >> 1];
        }
        lut_lds[2 * m] = sel[0];
        lut_lds[2 * m + 1] = sel[1];
    }

    const uint32_t dmax = (area_kb + (uint32_t)nwaves - 1u) / (uint32_t)nwaves;   // DMA instructions per wavefront
    auto issue = [&](int i) -> void {
        const BtRange g = bf_range(eb[i], eb[i + 1]);
        const uint32_t n = min(g.n, cap);
        uint8_t *buf = stage + (uint32_t)(i % 3) * area;
        for (uint32_t d = 0; d < dmax; ++d) {
            const uint32_t j = (uint32_t)wave + (uint32_t)nwaves * d;
            if (j >= area_kb) break;   // wave-uniform
            const uint32_t u = j * 64u + (uint32_t)lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(buf + j * 1024u), 16,
                                                     u < n ? (g.g0 + u) * 16u : 0xFFFFFFF0u, 0, 0, BT_NT);
        }
    };
    // Y of step i (ring): item (row j, column n) adds D[j][n] and D[8 + j][8 +
    // n] of every wavefront (lanes (j/4)*16 + n and 32 + (j/4)*16 + 8 + n,
    // register j % 4 in the 16x16 D layout), in wavefront order; one rounding
    // to fp16. Thread t takes item t / nwaves when t % nwaves == 0: the 64
    // items are spread over the wavefronts.
    auto write_step = [&](int i) -> void {
        if ((int)threadIdx.x % nwaves != 0) return;
        const int o = (int)threadIdx.x / nwaves, j = (o >> 3) & 7, n = o & 7;
        const int m = (s_begin + i) * 8 + j;
        if (n >= N || m >= M) return;
        const int k = j & 3, l1 = (j >> 2) * 16 + n, l2 = 32 + (j >> 2) * 16 + 8 + n;
        float sum = 0.f;
        for (int w = 0; w < nwaves; ++w) {
            const float *pw = part + ((i & 1) * nwaves + w) * 256 + k * 64;
            sum += pw[l1];
            sum += pw[l2];
        }
        Y[(int64_t)n * M + m] = __builtin_bit_cast(uint16_t, (_Float16)sum);
    };
    issue(0);
    bf_h8 xb[1][8];   // X of this lane's tile, loaded behind the first DMA (below)
    bt_v4i xg[1][8];  // the same in runs of the rows, before the transpose (XR: N > 4)
    constexpr bool x_runs = XR;

#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        if (i >= nstep) break;
        const uint64_t word = tile_ok ? words[i] : 0ull;
        const uint32_t seg = (uint32_t)__builtin_popcountll(word);
        uint32_t incl = seg;
        {
            const uint32_t u16 = (uint32_t)__shfl_up((int)incl, 16, 64);
            incl += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)incl, 32, 64);
            incl += q >= 2 ? u32 : 0u;
        }
        int32_t *wti = wt + i * BF_ROWS * BF8_WAVES;
        if (q == 3) wti[r * BF8_WAVES + wave] = (int32_t)incl;   // this wavefront's total for half row r
        if (i == 0) {
            // X of this lane's tile: column r & 7, as the B operands of the
            // tile's 8 MFMAs (column >= N, a tile past the half or past K:
            // zeros). Issued after the words and the first DMA so that neither
            // waits behind it; the decode is the first use.
            const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(X, (uint32_t)N * (uint32_t)K * 2u);
            const int n = row8;
            if constexpr (x_runs) {
                // at N > 4, in 64-byte runs of the rows (load j gives lane
                // group q granule 4 j + q of the wavefront's four tiles of
                // this half), handed out by the lane-group transpose before
                // the decode
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t gi = 4u * (uint32_t)j + (uint32_t)q;
                    const uint32_t tw2 = (uint32_t)(wave * 4) + (gi >> 3);
                    const uint32_t tt = (uint32_t)(kh * T2) + tw2;
                    const uint32_t k0 = tt * 64u + 8u * (gi & 7u);
                    const bool ok = n < N && tw2 < (uint32_t)T2 && tt < (uint32_t)T && k0 < (uint32_t)K;
                    xg[0][j] = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                                  xrs, ok ? ((uint32_t)n * (uint32_t)K + k0) * 2u : 0xFFFFFFF0u, 0, 0));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t k0 = (uint32_t)t * 64u + 8u * j;
                    const uint32_t off = (n < N && tile_ok && k0 < (uint32_t)K) ? ((uint32_t)n * (uint32_t)K + k0) * 2u
                                                                                : 0xFFFFFFF0u;
                    xb[0][j] = __builtin_bit_cast(bf_h8, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
                }
            }
        }
        bt_wait_vm(0);   // this wavefront's share of step i landed (nothing later in flight)
        if (i + 1 < nstep) issue(i + 1);
        bt_barrier_lds();   // everyone's share, every half-row total of step i, step i - 1's partials
        if (RING && i > 0) write_step(i - 1);

        const BtRange g = bf_range(eb[i], eb[i + 1]);
        // element index of the lane's first nonzero, counted from the step's first granule
        uint32_t pstart;
        {
            uint32_t pre[BF8_WAVES + 1];
            pre[0] = 0;
            const bt_v4i t0v = *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(wti + r * BF8_WAVES);
            const bt_v4i t1v = *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(wti + r * BF8_WAVES + 4);
            pre[1] = (uint32_t)t0v.x; pre[2] = pre[1] + (uint32_t)t0v.y;
            pre[3] = pre[2] + (uint32_t)t0v.z; pre[4] = pre[3] + (uint32_t)t0v.w;
            pre[5] = pre[4] + (uint32_t)t1v.x; pre[6] = pre[5] + (uint32_t)t1v.y;
            pre[7] = pre[6] + (uint32_t)t1v.z; pre[8] = pre[7] + (uint32_t)t1v.w;
            pstart = (hs[i] - (eb[i] & ~7u)) + pre[wave] + (incl - seg);
        }
        if constexpr (x_runs)
            if (i == 0) bf_x_transpose<1>(xg, xb);
        bf_f4 acc[1] = {bf_f4{0.f, 0.f, 0.f, 0.f}};
        if (g.n <= cap) {
            uint32_t p = min(pstart, 2u * (4u * g.n - 3u));   // a corrupt stream stays inside the staged granules
            p += bt_lds_addr(stage + (uint32_t)(i % 3) * area) >> 1;
            bf_contract_lds_ahead<1>(word, p, lut, xb, acc);
        } else {
            bf_contract<1>(word, pstart, BfWinGlobal{prs, 4u * g.g0}, lut, xb, acc);
        }
        // (ring: slot i % 2 was last read by step i - 2's sum, before this step's barrier)
        float *pw = part + ((RING ? (i & 1) : i) * nwaves + wave) * 256;
#pragma unroll
        for (int k = 0; k < 4; ++k) pw[k * 64 + lane] = acc[0][k];
    }
    bt_barrier_lds();
    if constexpr (RING) {
        write_step(nstep - 1);
    } else {
        // every step's Y, items over all the threads
        for (int o = threadIdx.x; o < nstep * 64; o += blockDim.x) {
            const int i = o >> 6, j = (o >> 3) & 7, n = o & 7;
            const int m = (s_begin + i) * 8 + j;
            if (n >= N || m >= M) continue;
            const int k = j & 3, l1 = (j >> 2) * 16 + n, l2 = 32 + (j >> 2) * 16 + 8 + n;
            float sum = 0.f;
            for (int w = 0; w < nwaves; ++w) {
                const float *pw = part + (i * nwaves + w) * 256 + k * 64;
                sum += pw[l1];
                sum += pw[l2];
            }
            Y[(int64_t)n * M + m] = __builtin_bit_cast(uint16_t, (_Float16)sum);
        }
    }
}

// Plan of the eight-row kernel, or false when it does not apply.
struct Bf8Plan {
    int nwaves;
    int nstep;   // step slots per workgroup (2, 4 or 8), a template argument
    int ring;    // partials in a ring of two step slots (NSTEP 8 only), a template argument
    unsigned grid;
    int sq, sr;
    uint32_t area_kb;
    size_t lds;
};

static bool bf8_plan(int64_t M, int64_t K, int64_t N, int64_t payload_bytes, Bf8Plan *p) {
    if (K <= 0 || K % 8 != 0 || (K + 63) / 64 > 64 || N < 1 || N > 8 || M <= 0) return false;
    const int64_t T = (K + 63) / 64, T2 = (T + 1) / 2;
    p->nwaves = (int)((T2 + 3) / 4);
    const int64_t steps = (M + 7) / 8;
    // staging per step: 1.2x the average step plus 2 KB, in KB (a larger
    // step reads its windows from global memory), capped at a dense step
    const int64_t avg = payload_bytes / std::max<int64_t>(steps, 1);
    const int64_t worst = 8 * T * 128 + 64;
    const int64_t est = std::min<int64_t>(worst, avg + avg / 5 + 2048) + 32;
    p->area_kb = (uint32_t)std::max<int64_t>(1, (est + 1023) / 1024);
    const auto lds_of = [&](int64_t per_wg, int nstep, bool ring) -> size_t {
        return 128 + (size_t)nstep * BF_ROWS * BF8_WAVES * 4 +
               (size_t)(ring ? std::min<int64_t>(per_wg, 2) : per_wg) * p->nwaves * 256 * 4 +
               (size_t)std::min<int64_t>(per_wg, 3) * p->area_kb * 1024;
    };
    // two steps per workgroup at least (the second streams in while the
    // first decodes), one workgroup per CU; two step slots when that
    // suffices (the prologue loads every slot's words: fewer loads ahead of
    // the first DMA). Up to 8 steps each when that keeps the grid to one
    // workgroup per CU and fits the LDS, else up to 4 in rounds (11008 x 4096
    // at N = 1: 24.0 us in 1.34 rounds of 4 steps, 8192 rows 13.5); with the
    // partials in a ring of two slots when only that fits and the rounds
    // would leave part of a round idle (5 to 7 steps; density 0.5: 24.7 ->
    // 20.2 us, N = 8 27.3 -> 21.7; at 8 steps the rounds do as well)
    int64_t grid = std::max<int64_t>(std::min<int64_t>((steps + 1) / 2, BF_CUS), (steps + 3) / 4);
    int nstep = (steps + grid - 1) / grid <= 2 ? 2 : 4;
    bool ring = false;
    const int64_t grid8 = std::max<int64_t>(std::min<int64_t>((steps + 1) / 2, BF_CUS), (steps + 7) / 8);
    const int64_t per8 = (steps + grid8 - 1) / grid8;
    if (per8 > 4 && grid8 <= BF_CUS) {
        if (lds_of(per8, 8, false) <= (size_t)BF_LDS_MAX) {
            grid = grid8;
            nstep = 8;
        } else if (per8 < 8 && lds_of(per8, 8, true) <= (size_t)BF_LDS_MAX) {
            grid = grid8;
            nstep = 8;
            ring = true;
        }
    }
    p->nstep = nstep;
    p->ring = ring;
    p->grid = (unsigned)grid;
    p->sq = (int)(steps / grid);
    p->sr = (int)(steps % grid);
    const int64_t per_wg = (steps + grid - 1) / grid;
    p->lds = lds_of(per_wg, nstep, ring);
    return p->lds <= (size_t)BF_LDS_MAX;
}

static void launch_bt8_f16(const Bf8Plan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                           const uint16_t *payload, uint32_t payload_bytes, int M, int K, const uint16_t *X, int N,
                           uint16_t *Y, hipStream_t stream) {
    // X in runs of the rows at N > 4 (4096 x 4096 at N = 8: 10.5 -> 9.5 us);
    // per-lane loads below (N = 1 and 4 measured 0.05 us faster that way)
#define BF8_LAUNCH(S, XR)                                                                                       \
    do {                                                                                                        \
        (void)hipFuncSetAttribute((const void *)k_bt8_f16<S, XR>, hipFuncAttributeMaxDynamicSharedMemorySize,  \
                                  (int)p.lds);                                                                  \
        hipLaunchKernelGGL((k_bt8_f16<S, XR>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream, offsets, M, K, \
                           p.sq, p.sr, bitmaps, X, N, payload, payload_bytes, Y, p.area_kb);                    \
    } while (0)
#define BF8_LAUNCH_R(S, XR)                                                                                         \
    do {                                                                                                            \
        (void)hipFuncSetAttribute((const void *)k_bt8_f16<S, XR, true>,                                             \
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);                          \
        hipLaunchKernelGGL((k_bt8_f16<S, XR, true>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream, offsets, M, \
                           K, p.sq, p.sr, bitmaps, X, N, payload, payload_bytes, Y, p.area_kb);                     \
    } while (0)
    if (p.nstep == 2) {
        if (N > 4) BF8_LAUNCH(2, true); else BF8_LAUNCH(2, false);
    } else if (p.nstep == 4) {
        if (N > 4) BF8_LAUNCH(4, true); else BF8_LAUNCH(4, false);
    } else if (!p.ring) {
        if (N > 4) BF8_LAUNCH(8, true); else BF8_LAUNCH(8, false);
    } else {
        if (N > 4) BF8_LAUNCH_R(8, true); else BF8_LAUNCH_R(8, false);
    }
#undef BF8_LAUNCH_R
#undef BF8_LAUNCH
}

struct BfPlan {
    int nwaves, nb;
    int psets;   // sets of per-wavefront partials (1 or 2)
    unsigned grid;
    int bq, br;
    uint32_t stage_bytes, nbuf;
    size_t lds;
};

// Fast-path constraints: one tile per lane (K <= 4096) and N <= 32.
static bool bf_supported(int64_t K, int64_t N) {
    return K > 0 && K % 8 == 0 && (K + 63) / 64 <= 4 * BF_MAX_WAVES && N >= 1 && N <= 32;
}

static bool bf_plan(int64_t M, int64_t K, int64_t N, int64_t payload_bytes, BfPlan *p) {
    if (!bf_supported(K, N) || M <= 0) return false;
    const int64_t T = (K + 63) / 64;
    p->nwaves = (int)((T + 3) / 4);
    p->nb = N <= 16 ? 1 : 2;
    const int64_t blocks = (M + BF_ROWS - 1) / BF_ROWS;
    const int64_t grid = std::max<int64_t>(std::min<int64_t>(blocks, BF_CUS), (blocks + BF_NBLK - 1) / BF_NBLK);
    p->grid = (unsigned)grid;
    p->bq = (int)(blocks / grid);
    p->br = (int)(blocks % grid);
    const int64_t per_wg = (blocks + grid - 1) / grid;
    const int64_t wg_per_cu = (grid + BF_CUS - 1) / BF_CUS;
    const int64_t budget = BF_LDS_MAX / wg_per_cu;
    const int64_t avg = payload_bytes / std::max<int64_t>(blocks, 1);
    const int64_t worst = (int64_t)BF_ROWS * T * 128 + 64;
    int64_t stage = std::min<int64_t>(worst, avg + avg / 5 + 2048) + 32;
    stage = (stage + 1023) / 1024 * 1024;
    // one set of partials when a workgroup owns a single block (the second
    // set only overlaps a block's partials with the previous block's sum),
    // or when two sets leave too little for two staging buffers
    int64_t psets = per_wg > 1 ? 2 : 1;
    int64_t fixed = 128 + 2 * BF_ROWS * BF_MAX_WAVES * 4 + psets * (int64_t)p->nwaves * p->nb * 256 * 4;
    int64_t nbuf = std::min<int64_t>((budget - fixed) / stage, per_wg);
    if (psets == 2 && nbuf < 2) {
        const int64_t fixed1 = fixed - (int64_t)p->nwaves * p->nb * 256 * 4;
        if (std::min<int64_t>((budget - fixed1) / stage, per_wg) >= 2) {
            psets = 1;
            fixed = fixed1;
            nbuf = std::min<int64_t>((budget - fixed) / stage, per_wg);
        }
    }
    p->psets = (int)psets;
    if (nbuf < std::min<int64_t>(2, per_wg)) {   // see the int4 plan
        stage = 0;
        nbuf = 1;
    }
    p->stage_bytes = (uint32_t)stage;
    p->nbuf = (uint32_t)nbuf;
    p->lds = (size_t)(fixed + nbuf * stage);
    return p->lds <= (size_t)budget;
}

template <int NB>
static void launch_bf_t(const BfPlan &p, const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                        uint32_t payload_bytes, int M, int K, const uint16_t *X, int N, uint16_t *Y,
                        hipStream_t stream) {
    (void)hipFuncSetAttribute((const void *)k_bt64_f16<NB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    hipLaunchKernelGGL((k_bt64_f16<NB>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream, bitmaps, offsets, payload,
                       payload_bytes, M, K, X, N, Y, p.stage_bytes, p.nbuf, p.bq, p.br, p.psets);
}

static void launch_bt64_f16(const BfPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                            const uint16_t *payload, uint32_t payload_bytes, int M, int K, const uint16_t *X, int N,
                            uint16_t *Y, hipStream_t stream) {
    if (p.nb == 1)
        launch_bf_t<1>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, stream);
    else
        launch_bf_t<2>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, stream);
}
