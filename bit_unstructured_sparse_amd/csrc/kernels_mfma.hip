// kernels_mfma.hip -- lane-per-tile decode + int8 MFMA contraction (gfx950).
//
// Work split. A workgroup owns 16 consecutive output rows (one 16-row MFMA
// block) and all of K. Its four wavefronts take the four K-quarters; inside a
// wavefront, lane l owns row r = l % 16 and lane group s = l / 16 owns a
// contiguous quarter of the wavefront's K-range, walked tile by tile. Each
// lane therefore decodes one whole 1 x 64 tile per step, and one step of the
// wavefront covers 16 rows x 4 tiles: four v_mfma_i32_16x16x64_i8, where
// MFMA i contracts positions 16i..16i+15 of every lane's tile (the K order
// inside an MFMA is free as long as A and B use the same one).
//
// Staging. Per 16-tile chunk, each wavefront copies the payload range of each
// of its 16 rows into its own LDS slot with buffer_load ... lds (LDS DMA):
// the row's range start and length are wave-uniform, so the copy costs no
// vector ALU work. Bitmap words are loaded straight into registers. Offsets
// are read once per lane per chunk; inside the chunk the running position is
// advanced by the popcount of each word (UnionSparse Sec. V-A: the offset is
// the prefix sum of the preceding tiles' popcounts).
//
// Decode (the hot step; UnionSparse Sec. VI-B and SPDP Sec. 4.2.1 do it one
// position per thread with a masked popcount; here it is done 8 positions at
// a time). For each byte b of the word (8 positions) the lane reads a 32-bit
// window of the next 8 payload nibbles from LDS (a funnel shift of two
// dwords), splits it into even and odd nibbles placed in the high half of
// each byte (x16 scaling, so no sign extension is needed), and builds the 8
// output bytes with two v_perm_b32 whose selectors come from a 256-entry LDS
// table indexed by b: selector byte = the rank of the position's nonzero
// among the byte's set bits, or "zero" for an unset bit.
//
// Activations. X stays int4 in memory; each lane converts the 64-column slab
// it needs into the same even/odd x16 byte order (one AND, or a shift and an
// AND, per 8 values). Products are therefore 256 x W x X; the int32 sums are
// exact while 256 * 64 * K < 2^31 (K < 2^17, checked on the host) and are
// shifted right by 8 at the end.

#define BSP_MF_ROWS 16                 // rows per workgroup (one MFMA row block)
#define BSP_MF_WAVES 4                 // wavefronts per workgroup (K quarters)
#ifndef BSP_MF_CHUNK
#define BSP_MF_CHUNK 16                // tiles per staged chunk of a wavefront
#endif
#define BSP_MF_TPL (BSP_MF_CHUNK / 4)  // tiles per lane per chunk
// LDS slot per row per chunk, in 16-byte units: up to 16 tiles x 32 bytes of
// payload, one unit for the start misalignment and one for the window that
// reads one dword past the last nonzero.
#define BSP_MF_SLOT_UNITS (BSP_MF_CHUNK * 2 + 2)
// Row slots sit BSP_MF_SLOT_PAD units apart beyond their size so that the 16
// rows of a wavefront start in different LDS banks.
#ifndef BSP_MF_SLOT_PAD
#define BSP_MF_SLOT_PAD 1
#endif
#define BSP_MF_SLOT_BYTES ((BSP_MF_SLOT_UNITS + BSP_MF_SLOT_PAD) * 16)
#define BSP_MF_WAVE_LDS (BSP_MF_ROWS * BSP_MF_SLOT_BYTES)
// The selector table is stored BSP_MF_LUT_COPIES times, interleaved entry by
// entry; lane l reads copy l % BSP_MF_LUT_COPIES, which spreads the lanes'
// random lookups over more LDS banks.
#ifndef BSP_MF_LUT_COPIES
#define BSP_MF_LUT_COPIES 1
#endif
#define BSP_MF_LUT_BYTES (256 * 8 * BSP_MF_LUT_COPIES)
// LDS layout: the selector table (one copy per workgroup, at LDS address 0)
// followed by one slot area per wavefront.
#define BSP_MF_WAVE_AREA BSP_MF_WAVE_LDS

typedef int bsp_v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void bsp_lds_void;
typedef __attribute__((address_space(3))) const uint32_t bsp_lds_u32;

// Selector table for one bitmap byte b: .x builds the bytes of the even
// positions 0,2,4,6 of the byte, .y those of the odd positions 1,3,5,7.
// Sources of the v_perm: S1 (selector 0..3) holds payload nibbles 0,2,4,6 of
// the window, S0 (selector 4..7) holds nibbles 1,3,5,7; 0x0C yields zero.
// Generated at compile time; entry b, copy c is dword pair
// (b * copies + c) of the table, the same layout the LDS copy uses.
struct BspMfLut {
    uint32_t w[256 * 2 * BSP_MF_LUT_COPIES];
};

constexpr BspMfLut bsp_mf_make_lut() {
    BspMfLut t{};
    for (uint32_t b = 0; b < 256; ++b) {
        uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu};
        uint32_t r = 0;
        for (int i = 0; i < 8; ++i) {
            if ((b >> i) & 1u) {
                const uint32_t src = (r & 1u) ? 4u + (r >> 1) : (r >> 1);
                const int half = i & 1, byte = i >> 1;
                sel[half] = (sel[half] & ~(0xFFu << (8 * byte))) | (src << (8 * byte));
                ++r;
            }
        }
        for (int c = 0; c < BSP_MF_LUT_COPIES; ++c) {
            t.w[2 * (b * BSP_MF_LUT_COPIES + c)] = sel[0];
            t.w[2 * (b * BSP_MF_LUT_COPIES + c) + 1] = sel[1];
        }
    }
    return t;
}

__device__ __attribute__((aligned(16))) const BspMfLut bsp_mf_lut_global = bsp_mf_make_lut();

// Decode of one tile, split in two so that all of a tile's LDS reads are in
// flight together before any of them is used:
//   fetch: for every byte group g, the selector pair of its byte b_g and the
//          two payload dwords holding nibbles q_g .. q_g+7, where q_g is the
//          tile's start position plus the popcount of the bytes before g;
//   build: funnel-shift the 8-nibble window, split it into even and odd
//          nibbles in the high half of each byte (x16, so no sign extension),
//          and place the bytes with two v_perm_b32. Output A[2g] holds
//          positions 8g+{0,2,4,6}, A[2g+1] positions 8g+{1,3,5,7}.
// q counts nibbles from the start of LDS.
struct BspMfFetch {
    uint2 sel[8];
    uint32_t w0[8], w1[8];
    uint32_t q[8];
};

__device__ __forceinline__ void bsp_mf_fetch(uint64_t word, uint32_t q, const uint2 *__restrict__ lut,
                                             BspMfFetch &f) {
    const uint32_t lo = (uint32_t)word, hi = (uint32_t)(word >> 32);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const uint32_t b = __builtin_amdgcn_ubfe(g < 4 ? lo : hi, 8 * (g & 3), 8);
        f.q[g] = q;
        f.sel[g] = lut[b];
        const bsp_lds_u32 *w = (const bsp_lds_u32 *)(uintptr_t)((q >> 1) & ~3u);
        f.w0[g] = w[0];
        f.w1[g] = w[1];
        q += __builtin_popcount(b);
    }
}

__device__ __forceinline__ void bsp_mf_build(const BspMfFetch &f, uint32_t A[16]) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        // v_alignbit_b32 uses only the low five bits of the shift: 4 * (q % 8)
        const uint32_t x = __builtin_amdgcn_alignbit(f.w1[g], f.w0[g], f.q[g] << 2);
        const uint32_t s_odd = x & 0xF0F0F0F0u;
        const uint32_t s_even = (x << 4) & 0xF0F0F0F0u;
        A[2 * g] = __builtin_amdgcn_perm(s_odd, s_even, f.sel[g].x);
        A[2 * g + 1] = __builtin_amdgcn_perm(s_odd, s_even, f.sel[g].y);
    }
}

// X slab for one (n, tile): 8 dwords of packed int4 -> 16 dwords of x16 int8
// in the decode's order (even positions, then odd positions, per 8 values).
__device__ __forceinline__ void bsp_mf_convert_x(const uint32_t d[8], uint32_t B[16]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        B[2 * q] = (d[q] << 4) & 0xF0F0F0F0u;
        B[2 * q + 1] = d[q] & 0xF0F0F0F0u;
    }
}

// Maximum wavefronts per workgroup: the workgroup splits K in chunks of
// BSP_MF_CHUNK tiles, one chunk per wavefront (more chunks loop).
#ifndef BSP_MF_MAX_WAVES
#define BSP_MF_MAX_WAVES 12
#endif

template <int NBLK>
__global__ __launch_bounds__(BSP_WAVE * BSP_MF_MAX_WAVES) void k_mfma_w4a4(
        const uint64_t *__restrict__ bitmaps, const uint32_t *__restrict__ offsets,
        const uint8_t *__restrict__ payload, uint32_t payload_bytes, int M, int K,
        const uint8_t *__restrict__ X, int N, int32_t *__restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t bsp_smem[];
    const int nwaves = blockDim.x / BSP_WAVE;
    const int wave = threadIdx.x / BSP_WAVE;
    const int lane = threadIdx.x % BSP_WAVE;
    const uint2 *lut = reinterpret_cast<const uint2 *>(bsp_smem);
    uint8_t *wave_lds = bsp_smem + BSP_MF_LUT_BYTES + wave * BSP_MF_WAVE_AREA;

    const int T = (K + 63) >> 6;
    const int m0 = blockIdx.x * BSP_MF_ROWS;
    const int r = lane & 15, s = lane >> 4;
    const int m = m0 + r;
    const bool row_ok = m < M;
    const int64_t rowg = (int64_t)min(m, M - 1) * T;
    const int xs = (K + 1) >> 1;     // X row stride in bytes (K % 8 == 0 on this path)
    const __amdgpu_buffer_rsrc_t prs = bsp_rsrc(payload, payload_bytes);
    const __amdgpu_buffer_rsrc_t xrs = bsp_rsrc(X, (uint32_t)(N * xs));

    bsp_v4i acc[NBLK];
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) acc[nb] = bsp_v4i{0, 0, 0, 0};

    // Selector table: global (L2-resident) -> registers, issued before any
    // other load; it goes to LDS behind one early workgroup barrier, long
    // before the payload arrives.
    constexpr int lut_units = BSP_MF_LUT_BYTES / 16;
    const __amdgpu_buffer_rsrc_t lrs = bsp_rsrc(&bsp_mf_lut_global, (uint32_t)sizeof(BspMfLut));
    bsp_v4i lut_part[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = (int)threadIdx.x + k * (int)blockDim.x;
        if (u < lut_units && (k == 0 || (int)blockDim.x < lut_units))
            lut_part[k] = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(lrs, u * 16, 0, 0));
    }
    bool table_ready = false;

    for (int c0 = wave * BSP_MF_CHUNK; c0 < T; c0 += nwaves * BSP_MF_CHUNK) {
        const int c1 = min(T, c0 + BSP_MF_CHUNK);
        // (1) the row's payload range for this chunk and this lane's start
        // position, issued first: the payload loads wait on them.
        const int ts0 = min(c1, c0 + s * BSP_MF_TPL), ts1 = min(c1, ts0 + BSP_MF_TPL);
        uint32_t nib0 = 0, nib1 = 0, lane_nib0 = 0;
        if (row_ok) {
            nib0 = offsets[rowg + c0];
            nib1 = offsets[rowg + c1];
            lane_nib0 = offsets[rowg + min(ts0, c1)];
        }
        // (2) loads that do not depend on the offsets: bitmap words and X slabs
        uint64_t words[BSP_MF_TPL];
#pragma unroll
        for (int i = 0; i < BSP_MF_TPL; ++i) words[i] = (row_ok && ts0 + i < ts1) ? bitmaps[rowg + ts0 + i] : 0ull;
        uint32_t xd[BSP_MF_TPL][NBLK][8];
#pragma unroll
        for (int i = 0; i < BSP_MF_TPL; ++i)
#pragma unroll
            for (int nb = 0; nb < NBLK; ++nb) {
                // a lane whose column n >= N reads past N*xs: the range check returns zeros;
                // a tile past the lane's range meets an all-zero A fragment, so its X is unused
                const uint32_t off = (uint32_t)((r + 16 * nb) * xs + (ts0 + i) * 32);
                const bsp_v4i v0 = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
                const bsp_v4i v1 = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off + 16, 0, 0));
                xd[i][nb][0] = v0.x; xd[i][nb][1] = v0.y; xd[i][nb][2] = v0.z; xd[i][nb][3] = v0.w;
                xd[i][nb][4] = v1.x; xd[i][nb][5] = v1.y; xd[i][nb][6] = v1.z; xd[i][nb][7] = v1.w;
            }
        if (!table_ready) {   // first chunk: publish the table (waits for its load only)
            bsp_v4i *lut_lds = reinterpret_cast<bsp_v4i *>(bsp_smem);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int u = (int)threadIdx.x + k * (int)blockDim.x;
                if (u < lut_units && (k == 0 || (int)blockDim.x < lut_units)) lut_lds[u] = lut_part[k];
            }
            __syncthreads();
            table_ready = true;
        }
        // (3) the payload: the 4 lanes of a row fetch its 16-byte units
        // s, s+4, s+8, ... straight into registers (all in flight together)
        const uint32_t u0 = nib0 >> 5;
        const uint32_t u1 = (nib1 >> 5) + 2u;
        // never more than the slot holds, whatever the offsets say
        const uint32_t nunits = (row_ok && u1 > u0) ? min(u1 - u0, (uint32_t)BSP_MF_SLOT_UNITS) : 0u;
        constexpr int kRounds = (BSP_MF_SLOT_UNITS + 3) / 4;
        bsp_v4i pu[kRounds];
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const uint32_t u = (uint32_t)(s + 4 * k);
            if (u < nunits) pu[k] = __builtin_bit_cast(bsp_v4i, __builtin_amdgcn_raw_buffer_load_b128(prs, (u0 + u) * 16, 0, 0));
        }
        // (4) registers -> LDS: this row's slot
        bsp_v4i *slot = reinterpret_cast<bsp_v4i *>(wave_lds + r * BSP_MF_SLOT_BYTES);
#pragma unroll
        for (int k = 0; k < kRounds; ++k) {
            const uint32_t u = (uint32_t)(s + 4 * k);
            if (u < nunits) slot[u] = pu[k];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's LDS writes landed
        __builtin_amdgcn_wave_barrier();

        // q: nibble position inside the workgroup's LDS (this wavefront's slot
        // base folded in, so the window address needs no extra add)
        const uint32_t slot_base = (uint32_t)(uintptr_t)(const bsp_lds_void *)(wave_lds + r * BSP_MF_SLOT_BYTES);
        uint32_t q = slot_base * 2u + lane_nib0 - (u0 << 5);
        if (!row_ok) q = slot_base * 2u;
#pragma unroll
        for (int i = 0; i < BSP_MF_TPL; ++i) {
            BspMfFetch f;                  // all 24 LDS reads of the tile in flight together
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
        __builtin_amdgcn_wave_barrier();   // the slot is rewritten by the next chunk
    }

    if (!table_ready) {   // no chunk for this wavefront: still publish its share of the table
        bsp_v4i *lut_lds = reinterpret_cast<bsp_v4i *>(bsp_smem);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int u = (int)threadIdx.x + k * (int)blockDim.x;
            if (u < lut_units && (k == 0 || (int)blockDim.x < lut_units)) lut_lds[u] = lut_part[k];
        }
        __syncthreads();
    }

    // --- reduce the wavefronts' K chunks through LDS, then write Y (x256 removed)
    __syncthreads();
    int32_t *red = reinterpret_cast<int32_t *>(bsp_smem + BSP_MF_LUT_BYTES);
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

static bool mfma_w4a4_supported(int64_t K) {
    return K % 8 == 0 && K < (1 << 17);
}

static void launch_mfma_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                             uint32_t payload_bytes, int M, int K, const uint8_t *X, int N, int32_t *Y,
                             hipStream_t stream) {
    const int T = (K + 63) / 64;
    // one chunk of BSP_MF_CHUNK tiles per wavefront when K allows
    const int nw = std::max(1, std::min(BSP_MF_MAX_WAVES, (T + BSP_MF_CHUNK - 1) / BSP_MF_CHUNK));
    const size_t lds = BSP_MF_LUT_BYTES + (size_t)nw * BSP_MF_WAVE_AREA;
    const dim3 block(BSP_WAVE * nw), grid((unsigned)((M + BSP_MF_ROWS - 1) / BSP_MF_ROWS));
    if (N <= 16) {
        hipFuncSetAttribute((const void *)k_mfma_w4a4<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k_mfma_w4a4<1>, grid, block, lds, stream, bitmaps, offsets, payload, payload_bytes,
                           M, K, X, N, Y);
    } else {
        hipFuncSetAttribute((const void *)k_mfma_w4a4<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k_mfma_w4a4<2>, grid, block, lds, stream, bitmaps, offsets, payload, payload_bytes,
                           M, K, X, N, Y);
    }
}
