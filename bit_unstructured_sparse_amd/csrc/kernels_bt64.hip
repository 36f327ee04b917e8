// kernels_bt64.hip -- block-staged bitmap decode + int8 MFMA contraction for
// the int4 x int4 -> int32 SpMM on gfx950 (CDNA4).
//
// Y = W_sparse * X with W in the BT64 stream (UnionSparse, Sec. V-A, one area
// per 1 x 64 tile: occupancy word, prefix offsets, packed nonzeros) and X a
// skinny K x N int4 matrix. The pages decode position-per-thread with a masked
// popcount (UnionSparse Sec. VI-B, SPDP Sec. 4.2.1) into tensor-core
// fragments; here the same arithmetic is reorganised for gfx950:
//
// Work split. Rows are cut into blocks of 16 (the A-row count of
// v_mfma_i32_16x16x64_i8). A workgroup is resident on one CU for the whole
// kernel and owns a contiguous run of at most BT_NBLK(TPL) blocks. Its
// wavefront w owns the tile range [4*TPL*w, 4*TPL*(w+1)) of every block, and
// inside it lane l = r + 16 q owns row r and the TPL consecutive tiles
// 4*TPL*w + TPL*q ... A step decodes one whole 1 x 64 tile per lane and issues
// four MFMAs; MFMA j contracts positions 16j .. 16j+15 of every lane's tile
// against the matching X slice (the K order inside one MFMA is free as long as
// A and B use the same one).
//
// Loads. Everything is requested up front: the block-boundary offsets (scalar
// loads), every block's bitmap words for this lane, this lane's X slices (kept
// in VGPRs for the whole launch) and the payload of as many blocks as the LDS
// ring holds. A block's payload is one contiguous range of the stream (tiles
// are in row-major order), so it needs only its two boundary offsets; it is
// moved by LDS DMA (16-byte granules, no VGPRs). Each lane's start inside it
// is the block start plus bitmap popcounts (the offset definition of
// Sec. V-A), exchanged across wavefronts through LDS at the block's barrier.
// Blocks are decoded in order while later ones are still in flight; a
// buffer is refilled once the block in it has been decoded. A block whose
// payload does not fit a buffer reads its windows from global memory instead
// (slower, same result).
//
// Windows. The 8 nibbles a step needs start at an arbitrary nibble p of the
// block's stream and span the two dwords p >> 3 and (p >> 3) + 1; one
// ds_read2_b32 fetches both and a funnel shift by 4 * (p & 7) aligns them.
//
// Decode of 8 positions (one byte b of the word). The window is split into
// even and odd nibbles placed in the high half of each byte (so a byte holds
// 16 * value and needs no sign extension) and two v_perm_b32 place them; the
// selector pair comes from a 256-entry LDS table indexed by b: for each of the
// byte's positions, the rank of its nonzero among the byte's set bits, or
// "zero". Output dword 2k holds positions 8k+{0,2,4,6}, dword 2k+1 positions
// 8k+{1,3,5,7}: the order a packed X dword splits into with one AND (odd k)
// or a shift and an AND (even k), which is the B operand order.
//
// Products are 256 * w * x; each wavefront's partial sum is shifted right by 8
// (exact) before the wavefronts' partials are added, so no int32 sum can
// overflow under the API's K bound.

#define BT_ROWS 16                      // rows per block (MFMA A rows)
#define BT_LUT_COPIES 16               // selector-table copies in LDS (lane l reads copy l % 16)
#define BT_LUT_BYTES (2048 * BT_LUT_COPIES)   // 256 entries x 8 bytes per copy
#define BT_LDS_MAX (160 * 1024)
#define BT_CUS 256
// Cache policy of the payload DMAs (and of the streaming kernel's bitmap
// words): non-temporal. Each of these bytes is read once per launch, by one
// workgroup, in whole 64-byte lines; the hint keeps them from displacing X and
// the other lines the launch reuses. Loads whose lines are shared between
// wavefronts or instructions (X, the ring kernel's 8-byte words, the fp16
// half-row starts) keep the default policy: marked non-temporal they were
// re-fetched and measured slower.
#define BT_NT 2

// Blocks one workgroup can own: every block's words stay in VGPRs (TPL words per lane).
#define BT_NBLK(TPL) (8 / (TPL))
// Threads per workgroup at most: 8 wavefronts (<= 256 VGPRs each).
#define BT_WG_THREADS(TPL) 512

typedef int bt_v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void bt_lds_void;
typedef __attribute__((address_space(3))) const uint64_t bt_lds_u64;
typedef __attribute__((address_space(3))) const uint32_t bt_lds_u32;
typedef __attribute__((address_space(3))) const bt_v4i bt_lds_v4i;

// Selector table: entry b (a bitmap byte) is the v_perm_b32 selector pair that
// scatters the byte's nonzeros to their positions. The perm's sources are
// S0 = odd-rank nibbles (selector 4..7) and S1 = even-rank nibbles (0..3);
// selector 0x0C yields a zero byte. Position p of the byte goes to byte p >> 1
// of selector p & 1; its source is the rank of its nonzero among the byte's
// set bits. Computed in registers (no table in memory to wait for).
__device__ __forceinline__ uint2 bt_lut_entry(uint32_t b) {
    uint32_t sel[2] = {0x0C0C0C0Cu, 0x0C0C0C0Cu};
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t rank = (uint32_t)__builtin_popcount(b & ((1u << p) - 1u));
        const uint32_t src = (rank >> 1) | ((rank & 1u) << 2);
        const uint32_t sh = 8u * (uint32_t)(p >> 1);
        const uint32_t upd = (sel[p & 1] & ~(0xFFu << sh)) | (src << sh);
        sel[p & 1] = ((b >> p) & 1u) ? upd : sel[p & 1];
    }
    return uint2{sel[0], sel[1]};
}

// LDS byte address of a pointer into dynamic shared memory.
__device__ __forceinline__ uint32_t bt_lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const bt_lds_void *)p;
}

// One aligned 8-byte LDS read (ds_read_b64) at byte address a, as (lo, hi).
__device__ __forceinline__ uint2 bt_lds_pair(uint32_t a) {
    const uint64_t v = *(bt_lds_u64 *)(uintptr_t)a;
    return uint2{(uint32_t)v, (uint32_t)(v >> 32)};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bt_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(n) for a run-time n (the instruction takes an immediate):
// waits until at most n vector-memory operations of this wavefront are
// outstanding. n above the counter's range (63) waits for n = 63.
__device__ __forceinline__ void bt_wait_vm(uint32_t n) {
#define BT_W(c) case c: __builtin_amdgcn_s_waitcnt(((c) & 15) | (((c) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
#define BT_W8(c) BT_W(c) BT_W(c + 1) BT_W(c + 2) BT_W(c + 3) BT_W(c + 4) BT_W(c + 5) BT_W(c + 6) BT_W(c + 7)
    switch (n < 63u ? n : 63u) {
        BT_W8(0) BT_W8(8) BT_W8(16) BT_W8(24) BT_W8(32) BT_W8(40) BT_W8(48) BT_W8(56)
    }
#undef BT_W8
#undef BT_W
}

// Workgroup barrier for LDS traffic only: waits for this wavefront's LDS
// operations, not for its outstanding global loads and payload DMAs (whose
// completion the caller establishes with bt_wait_vm where it needs it).
__device__ __forceinline__ void bt_barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Range of the X buffer resource: its N rows of xs bytes, rounded up to a
// whole dword. The hardware checks the range per dword, so a last dword only
// partly inside N * xs would read as zero; the dword holding the buffer's last
// byte lies in the same page as that byte, and its bytes past the end meet
// zero bits of the last tile (columns >= K).
__device__ __forceinline__ uint32_t bt_x_range(int N, uint32_t xs) {
    return ((uint32_t)N * xs + 3u) & ~3u;
}

// Output stage of the int4 MFMA kernels. Y receives the int32 sums; with
// the dequant epilogue (Yh set) Yh receives instead, for output row m and
// column n, fp16(fp32(fp32(y) * sw[m]) * sx[n]): the int32 sum converted to
// fp32, times the output channel's scale, times the token's scale, each
// product rounded to nearest even in fp32, then one round to nearest even to
// fp16 (the Dequant step that follows the SpMM in UnionSparse, Fig. 2, fused
// into the kernel's final write).
struct BtEpi {
    uint16_t *Yh;
    const float *sw;
    const float *sx;
};

__device__ __forceinline__ uint16_t bt_dequant(int32_t v, float sw, float sx) {
    const float a = (float)v * sw;
    float b = a * sx;
    // b is rounded to fp32 and only then converted: left to itself the
    // compiler turns the second product and the conversion into one
    // mixed-precision multiply that rounds once, from the exact product
    asm volatile("" : "+v"(b));
    return bsp_f2h(b);
}

__device__ __forceinline__ void bt_store_y1(int32_t *Y, const BtEpi &e, int M, int n, int m, int32_t v) {
    const int64_t at = (int64_t)n * M + m;
    if (e.Yh != nullptr)
        e.Yh[at] = bt_dequant(v, e.sw[m], e.sx[n]);
    else
        Y[at] = v;
}

// Rows m .. m+3 of column n (those below M).
__device__ __forceinline__ void bt_store_y4(int32_t *Y, const BtEpi &e, int M, int n, int m, bt_v4i v) {
    const int64_t at = (int64_t)n * M + m;
    const bool whole = m + 4 <= M && (M & 3) == 0;
    if (e.Yh != nullptr) {
        const float sx = e.sx[n];
        if (whole && ((uintptr_t)e.Yh & 7u) == 0 && ((uintptr_t)e.sw & 15u) == 0) {
            const float4 w = *reinterpret_cast<const float4 *>(e.sw + m);
            const uint32_t lo = (uint32_t)bt_dequant(v.x, w.x, sx) | ((uint32_t)bt_dequant(v.y, w.y, sx) << 16);
            const uint32_t hi = (uint32_t)bt_dequant(v.z, w.z, sx) | ((uint32_t)bt_dequant(v.w, w.w, sx) << 16);
            *reinterpret_cast<uint2 *>(e.Yh + at) = uint2{lo, hi};
        } else {
            const int32_t a[4] = {v.x, v.y, v.z, v.w};
            for (int k = 0; k < 4 && m + k < M; ++k) e.Yh[at + k] = bt_dequant(a[k], e.sw[m + k], sx);
        }
        return;
    }
    if (whole && ((uintptr_t)Y & 15u) == 0) {
        *reinterpret_cast<bt_v4i *>(Y + at) = v;
    } else {
        const int32_t a[4] = {v.x, v.y, v.z, v.w};
        for (int k = 0; k < 4 && m + k < M; ++k) Y[at + k] = a[k];
    }
}

// 16 bytes of X at byte offset off. X rows start on a 4-byte boundary when
// K % 8 == 0 (XU false): one 16-byte load. Otherwise (XU true) the dwords
// around the bytes are loaded from the 4-byte boundary below off and the
// bytes are funnel-shifted into place (v_alignbyte_b32). An offset past the
// buffer reads zeros either way.
template <bool XU>
__device__ __forceinline__ bt_v4i bt_load_x16(__amdgpu_buffer_rsrc_t xrs, uint32_t off) {
    if constexpr (!XU) {
        return __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
    } else {
        const uint32_t a = off & ~3u, sh = off & 3u;
        const bt_v4i d = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, a, 0, 0));
        const uint32_t e = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(xrs, a + 16u, 0, 0);
        return bt_v4i{(int)__builtin_amdgcn_alignbyte((uint32_t)d.y, (uint32_t)d.x, sh),
                      (int)__builtin_amdgcn_alignbyte((uint32_t)d.z, (uint32_t)d.y, sh),
                      (int)__builtin_amdgcn_alignbyte((uint32_t)d.w, (uint32_t)d.z, sh),
                      (int)__builtin_amdgcn_alignbyte(e, (uint32_t)d.w, sh)};
    }
}

// X of a wavefront's 4 TPL consecutive tiles (lane group q owns tiles
// q TPL .. q TPL + TPL - 1 of them) is 8 TPL contiguous 16-byte granules of
// each X row. Load i (i < 2 TPL) gives lane group q granule 4 i + q, so one
// load covers 64-byte runs of 16 rows; slices loaded lane by lane touch one
// line per lane instead, and the line requests, not the bytes, bound how
// fast X comes in. Columns n >= N and tiles >= T read zeros.
template <int NB, int TPL, bool XU>
__device__ __forceinline__ void bt_load_x_runs(__amdgpu_buffer_rsrc_t xrs, int r, int q, int wave, int T, int N,
                                               uint32_t xs, bt_v4i (&xg)[NB][2 * TPL]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n = r + 16 * nb;
#pragma unroll
        for (int i = 0; i < 2 * TPL; ++i) {
            const uint32_t gi = 4u * (uint32_t)i + (uint32_t)q;
            const uint32_t tt = (uint32_t)(wave * 4 * TPL) + (gi >> 1);
            const uint32_t off = (n < N && tt < (uint32_t)T) ? (uint32_t)n * xs + tt * 32u + (gi & 1u) * 16u : 0xFFFFFFE0u;
            xg[nb][i] = bt_load_x16<XU>(xrs, off);
        }
    }
}

// The granules of bt_load_x_runs -> each lane's own slices. With G = 2 TPL
// granules per lane and E = G / 4, element (q, s) = loads s E .. s E + E - 1
// of lane group q = the granules of group s taken by group q. A 4 x 4
// transpose over (q, s) gives group q the elements (s, q): its granule j is
// load (j / 4) of element j % 4. Two stages of swaps between lane groups:
// q ^ 2 (the 32-lane swap exchanges the upper half of its first operand with
// the lower half of its second) on elements s and s + 2, then q ^ 1 (the
// 16-lane swap exchanges the odd rows of the first with the even rows of the
// second) on elements 2u and 2u + 1. Every lane must be active.
template <int NB, int TPL>
__device__ __forceinline__ void bt_x_runs_to_slices(bt_v4i (&xg)[NB][2 * TPL], uint32_t (&xw)[NB][TPL][8]) {
    constexpr int E = TPL / 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < E; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const auto w = __builtin_amdgcn_permlane32_swap((unsigned)xg[nb][s * E + e][d],
                                                                    (unsigned)xg[nb][(s + 2) * E + e][d], false, false);
                    xg[nb][s * E + e][d] = (int)w[0];
                    xg[nb][(s + 2) * E + e][d] = (int)w[1];
                }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const auto w = __builtin_amdgcn_permlane16_swap((unsigned)xg[nb][2 * u * E + e][d],
                                                                    (unsigned)xg[nb][(2 * u + 1) * E + e][d], false, false);
                    xg[nb][2 * u * E + e][d] = (int)w[0];
                    xg[nb][(2 * u + 1) * E + e][d] = (int)w[1];
                }
#pragma unroll
        for (int k = 0; k < TPL; ++k) {
            const bt_v4i v0 = xg[nb][((2 * k) % 4) * E + (2 * k) / 4];
            const bt_v4i v1 = xg[nb][((2 * k + 1) % 4) * E + (2 * k + 1) / 4];
            xw[nb][k][0] = v0.x; xw[nb][k][1] = v0.y; xw[nb][k][2] = v0.z; xw[nb][k][3] = v0.w;
            xw[nb][k][4] = v1.x; xw[nb][k][5] = v1.y; xw[nb][k][6] = v1.z; xw[nb][k][7] = v1.w;
        }
    }
}

// Decode of one tile word into 16 dwords of x16 int8 (A operand of 4 MFMAs).
// win(p) returns the two payload dwords holding values p .. p+7 as (lo, hi).
// WB is the width of a stored value: 4 (int4 weights: each byte of the A
// operand is 16 w) or 2 (int2 weights, W2A4: the 16 bits of the window are
// spread to one 4-bit group per byte first, and each byte is 64 w).
// lut_base is the LDS address of this lane's copy of the selector table: the
// copies are interleaved entry by entry (entry b of copy c at (16 b + c) * 8),
// so the 16 lanes that read one copy each cannot conflict with one another.
template <class Win, int WB = 4>
__device__ __forceinline__ void bt_decode_tile(uint64_t word, uint32_t p, const Win &win, uint32_t lut_base,
                                               uint32_t A[16]) {
    const uint32_t lo = (uint32_t)word, hi = (uint32_t)(word >> 32);
    uint2 sel[8];
    uint2 d[8];
    uint32_t pk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t b = __builtin_amdgcn_ubfe(k < 4 ? lo : hi, 8 * (k & 3), 8);
        sel[k] = bt_lds_pair(lut_base + b * (8u * BT_LUT_COPIES));
        pk[k] = p;
        d[k] = win(p);
        p = (uint32_t)__builtin_popcount(b) + p;   // v_bcnt_u32_b32 with accumulate
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t s_odd, s_even;
        if constexpr (WB == 4) {
            const uint32_t x = __builtin_amdgcn_alignbit(d[k].y, d[k].x, pk[k] << 2);
            s_odd = x & 0xF0F0F0F0u;
            s_even = (x << 4) & 0xF0F0F0F0u;
        } else {
            uint32_t t = __builtin_amdgcn_alignbit(d[k].y, d[k].x, pk[k] << 1) & 0xFFFFu;
            t = (t | (t << 8)) & 0x00FF00FFu;
            t = (t | (t << 4)) & 0x0F0F0F0Fu;     // byte i: values 2i (bits 0-1) and 2i+1 (bits 2-3)
            s_odd = (t << 4) & 0xC0C0C0C0u;
            s_even = (t << 6) & 0xC0C0C0C0u;
        }
        A[2 * k] = __builtin_amdgcn_perm(s_odd, s_even, sel[k].x);
        A[2 * k + 1] = __builtin_amdgcn_perm(s_odd, s_even, sel[k].y);
    }
}

// Window source: the staged stream in LDS.
template <int WB = 4>
struct BtWinLdsT {
    // p counts values from 8 / WB times the staging buffer's LDS address (a
    // multiple of 16 bytes), so the dword holding value p sits at LDS byte
    // address (p >> (WB == 4 ? 1 : 2)) & ~3; the two dwords come from one
    // ds_read2_b32
    __device__ __forceinline__ uint2 operator()(uint32_t p) const {
        const bt_lds_u32 *q = (const bt_lds_u32 *)(uintptr_t)((p >> (WB == 4 ? 1 : 2)) & ~3u);
        return uint2{q[0], q[1]};
    }
};
using BtWinLds = BtWinLdsT<4>;

// Window source: global memory through a range-checked buffer resource
// (p counts values from payload dword d0).
template <int WB = 4>
struct BtWinGlobalT {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t d0;
    __device__ __forceinline__ uint2 operator()(uint32_t p) const {
        const uint32_t off = (d0 + (p >> (WB == 4 ? 3 : 4))) * 4u;
        return uint2{(uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0),
                     (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, off + 4u, 0, 0)};
    }
};

using BtWinGlobal = BtWinGlobalT<4>;

// X slice of one tile for one MFMA j: packed dwords x0 (k 0..7) and x1
// (k 8..15) -> B dwords {even k of x0, odd k of x0, even k of x1, odd k of x1}
// in the same x16 form as A.
__device__ __forceinline__ bt_v4i bt_b_operand(uint32_t x0, uint32_t x1) {
    return bt_v4i{(int)((x0 << 4) & 0xF0F0F0F0u), (int)(x0 & 0xF0F0F0F0u), (int)((x1 << 4) & 0xF0F0F0F0u),
                  (int)(x1 & 0xF0F0F0F0u)};
}

// Window positions of a tile as counted: p unchanged.
struct BtTileSame {
    __device__ __forceinline__ uint32_t operator()(uint32_t p) const { return p; }
};

// Decode + contract the lane's TPL tiles of one block. xb holds the lane's
// B operands (column r + 16 nb, tiles t0 .. t0+TPL-1, MFMA j), built once.
// tile(p) maps the stream position of a tile's first nonzero to the position
// its windows are read from.
template <int NB, int TPL, class Win, class Tile = BtTileSame, int WB = 4>
__device__ __forceinline__ void bt_contract(const uint64_t (&words)[TPL], uint32_t p, const Win &win,
                                            uint32_t lut_base, const bt_v4i (&xb)[NB][TPL][4],
                                            bt_v4i (&acc)[NB], const Tile &tile = Tile{}) {
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
        uint32_t A[16];
        bt_decode_tile<Win, WB>(words[i], tile(p), win, lut_base, A);
        p += (uint32_t)__builtin_popcountll(words[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bt_v4i a = {(int)A[4 * j], (int)A[4 * j + 1], (int)A[4 * j + 2], (int)A[4 * j + 3]};
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xb[nb][i][j], acc[nb], 0, 0, 0);
        }
    }
}

// Payload range of a block in 16-byte granules: [g0, g0 + n) covers its
// values (32 per granule for int4, 64 for int2) plus one granule for the
// windows that read past the last nonzero.
struct BtRange {
    uint32_t g0, n;
};
template <int WB = 4>
__device__ __forceinline__ BtRange bt_range(uint32_t nibA, uint32_t nibB) {
    constexpr uint32_t S = WB == 4 ? 5 : 6;
    const uint32_t g0 = nibA >> S;
    const uint32_t g1 = (nibB >= nibA ? (nibB + (1u << S) - 1u) >> S : g0) + 1u;
    return BtRange{g0, g1 - g0};
}

// LDS layout (bytes):
//   [row totals NBLK x 16 x 8 ints][sums 3 x NB x 256 ints][selector table copies]
//   [nbuf staging buffers of stage_bytes]
// Workgroup g owns blocks [g*bq + min(g, br), ...): bq or bq + 1 of them.
// XU: X rows are not on a 4-byte boundary (K % 8 != 0).
// STG: staggered staging. Rows whose length is a multiple of 64 B put the
// same tile of the 16 rows of a block on the same LDS banks (every row keeps
// the same count when each output row is pruned on its own). Staggered, DMA
// instruction j of a block stores its 1 KB with granules 61 j .. 61 j + 63 of
// the stream: each run of 61 granules is followed by the first 3 of the next
// (a tile's windows reach < 48 B past its first nonzero, so they stay inside
// the instruction of its start), and every 61 granules the stream moves 48 B
// further round the banks, so equal rows no longer line up.
// WB: width of a stored weight value (4: int4; 2: int2, the W2A4 variant,
// unstaggered).
#define BT_R61_RUN 61u
#define BT_R61_MAG 2200291u   // ceil(2^32 / (61 * 32)): umulhi(p, MAG) = p / 1952 for p < 2^20
// NBLK: blocks per workgroup, at most (8 / TPL; 8 at TPL 2 past 1024 blocks,
// 4 at TPL 4 and NB 1 past 512).
template <int NB, int TPL, bool XU, bool STG, int WB = 4, int NBLK = BT_NBLK(TPL)>
// (The arguments the first loads need come first: they are the ones a
// kernel-argument preload would place in registers.)
__global__ __launch_bounds__(BT_WG_THREADS(TPL)) void k_bt64_w4a4(
        const uint32_t *__restrict__ offsets, int M, int K, int bq, int br, const uint64_t *__restrict__ bitmaps,
        const uint8_t *__restrict__ X, int N, const uint8_t *__restrict__ payload, uint32_t payload_bytes,
        int32_t *__restrict__ Y, uint32_t stage_bytes, uint32_t nbuf, int one_pass, uint16_t *Yh, const float *sw,
        const float *sx) {
    static_assert(WB == 4 || (WB == 2 && !STG), "staggered staging is for int4 streams");
    const BtEpi epi{Yh, sw, sx};
    constexpr int WC = BT_WG_THREADS(TPL) / 64;          // row-total columns: wavefronts, at most
    constexpr uint32_t VPB = 8 / WB;                     // values per payload byte
    constexpr int PS = WB == 4 ? 8 : 10;                 // log2 of the A x B operand scale
    extern __shared__ __attribute__((aligned(16))) uint8_t bt_smem[];
    const int nwaves = blockDim.x >> 6;
    // the wavefront index is uniform: keep it (and the loops over it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int T = (K + 63) >> 6;
    const int gid = (int)blockIdx.x;
    const int b_begin = gid * bq + min(gid, br);
    const int nblk = bq + (gid < br ? 1 : 0);           // 1 .. NBLK
    const int t0 = (wave * 4 + q) * TPL;                 // first tile of this lane
    const uint32_t xs = ((uint32_t)K + 1u) >> 1;        // X row stride in bytes

    int32_t *wt = reinterpret_cast<int32_t *>(bt_smem);                                 // [NBLK][16][8]
    int32_t *sums = wt + NBLK * BT_ROWS * WC;                                            // [3][NB*256]
    uint8_t *lut_lds8 = reinterpret_cast<uint8_t *>(sums + 3 * NB * 256);
    uint8_t *stage = lut_lds8 + BT_LUT_BYTES;
    const uint32_t lut_base = bt_lds_addr(lut_lds8) + (uint32_t)(lane % BT_LUT_COPIES) * 8u;
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(payload, payload_bytes);

    // every kernel argument into SGPRs now, in the first batch of argument
    // loads: one loaded after the boundary offsets below would make its first
    // use wait for those too (scalar loads complete out of order)
    asm volatile("" ::"s"(bitmaps), "s"(payload), "s"(X), "s"(Y), "s"(N), "s"(stage_bytes), "s"(nbuf),
                 "s"(payload_bytes));

    // (1) block boundaries (wave-uniform scalar loads), before anything else:
    // the payload DMA waits for them
    uint32_t nib[NBLK + 1];
#pragma unroll
    for (int i = 0; i <= NBLK; ++i) {
        const int b = b_begin + (i < nblk ? i : nblk);
        nib[i] = offsets[(int64_t)min(b * BT_ROWS, M) * T];
    }
    // keep these loads issued here, ahead of the vector loads below (without
    // this the compiler sinks them to their first use, behind every wait)
    asm volatile("" ::: "memory");

    // (2) loads that need no offsets: this lane's X slices and every
    // block's bitmap words. Then the B operands are built (waiting for X
    // only), and then, once the offsets are in, the payload DMA of the first
    // nbuf blocks, each into staging buffer i % nbuf (its granules in stream
    // order, 1 KB = 64 lanes x 16 bytes per instruction; range checks of raw
    // buffer loads cover the per-lane offset only, so every offset is in the
    // per-lane operand). A block that does not fit is not staged: it reads
    // its windows from global memory.
    uint32_t vm_issued = 0;           // vector-memory operations issued so far by this wavefront
    // this lane's X slices, once for all blocks (column n >= N or tile >= T: zeros)
    uint32_t xw[NB][TPL][8];
    bt_v4i xg[NB][2 * TPL];           // X granules as loaded, in runs of 16 rows
    bt_load_x_runs<NB, TPL, XU>(bt_rsrc(X, bt_x_range(N, xs)), r, q, wave, T, N, xs, xg);
    vm_issued += 2 * NB * TPL;
    const int m_first = b_begin * BT_ROWS;
    const int wg_rows = min(nblk * BT_ROWS, M - m_first);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(bitmaps + (int64_t)m_first * T, (uint32_t)wg_rows * (uint32_t)T * 8u);
    uint64_t words[NBLK][TPL];
    // two consecutive tiles per 16-byte load (one per 8-byte load at TPL 8,
    // where the wider form costs registers)
    constexpr int WPL = TPL >= 8 ? 1 : 2;   // words per load
    // No select on the offsets (the compiler turns one into branches with a
    // wait in each): a row past the workgroup's range is past the end of the
    // buffer and reads zeros, and a tile past the row's end is cleared before
    // use.
    auto load_words = [&](int i) -> void {
        const int rr = i * BT_ROWS + r;   // row inside the workgroup's range
#pragma unroll
        for (int k = 0; k < TPL; k += WPL) {
            const uint32_t off = ((uint32_t)rr * (uint32_t)T + (uint32_t)(t0 + k)) * 8u;
            if constexpr (WPL == 2) {
                const bt_v4i v = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0));
                // a tile past T is cleared where the block is decoded: a select
                // here would wait for the load right away
                words[i][k] = ((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x;
                words[i][k + 1] = ((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z;
            } else {
                words[i][k] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off, 0, 0));
            }
        }
    };

    // every block slot is loaded, used or not (a slot past nblk reads
    // zeros): the compiler can then count the loads still in flight
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
        load_words(i);
        vm_issued += TPL / WPL;
    }
    // zero the sum buffers (first added to after the first block's barrier)
    for (int o = threadIdx.x; o < 3 * NB * 256; o += blockDim.x) sums[o] = 0;
    bt_x_runs_to_slices<NB, TPL>(xg, xw);
    // B operands of this lane's tiles, in the even/odd x16 order of the decode;
    // pinned so that they are built once, not rebuilt in every block
    bt_v4i xb[NB][TPL][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int k = 0; k < TPL; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xb[nb][k][j] = bt_b_operand(xw[nb][k][2 * j], xw[nb][k][2 * j + 1]);
                if constexpr (NBLK > 1) asm volatile("" : "+v"(xb[nb][k][j]));
            }

    // every block's segment popcounts (inclusive prefix over the lane groups
    // q of a row: lanes r, r+16, r+32, r+48) and this wavefront's row totals
    uint32_t seg[NBLK], incl[NBLK];
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
#pragma unroll
        for (int k = 0; k < TPL; ++k)
            if (t0 + k >= T) words[i][k] = 0;   // tiles past the row's end
        seg[i] = 0;
#pragma unroll
        for (int k = 0; k < TPL; ++k) seg[i] += (uint32_t)__builtin_popcountll(words[i][k]);
        uint32_t c = seg[i];
        const uint32_t u16 = (uint32_t)__shfl_up((int)c, 16, 64);
        c += q >= 1 ? u16 : 0u;
        const uint32_t u32 = (uint32_t)__shfl_up((int)c, 32, 64);
        c += q >= 2 ? u32 : 0u;
        incl[i] = c;
        if (q == 3) wt[(i * BT_ROWS + r) * WC + wave] = (int32_t)c;   // this wavefront's total for row r
    }

    // the payload DMA of the first blocks. It comes after every use of the
    // earlier loads: a wait for one of those after a loop of DMA issues would
    // have to wait for the DMAs too (the counter is in order, the loop's
    // length unknown to the compiler)
    uint32_t vm_mark[NBLK];
    constexpr uint32_t RUN = STG ? BT_R61_RUN : 64u;   // stream granules per 1 KB DMA instruction
    auto fits = [&](int i) -> bool {
        const BtRange g = bt_range<WB>(nib[i], nib[i + 1]);
        return (g.n + RUN - 1u) / RUN * 1024u <= stage_bytes;
    };
    auto issue_block = [&](int i) -> void {
        if (fits(i)) {
            const BtRange g = bt_range<WB>(nib[i], nib[i + 1]);
            uint8_t *buf = stage + (uint32_t)(i % (int)nbuf) * stage_bytes;
            // lane 0 of every instruction stores a granule of the block, so
            // each one issues (and counts)
            const uint32_t n_ins = (g.n + RUN - 1u) / RUN;
            for (uint32_t j = (uint32_t)wave; j < n_ins; j += (uint32_t)nwaves) {
                const uint32_t u = j * RUN + (uint32_t)lane;
                if (u < g.n)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(buf + j * 1024u), 16,
                                                             (g.g0 + u) * 16u, 0, 0, BT_NT);
                ++vm_issued;
            }
        }
        vm_mark[i] = vm_issued;
    };
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
        vm_mark[i] = vm_issued;   // the words; staging the block raises it
        if (i < nblk && i < (int)nbuf) issue_block(i);
    }

    // the selector table's copies, computed while the payload is in flight:
    // entry b of copy c at LDS slot 16 b + c (8 bytes); item v covers entry
    // v % 256, copies 8 (v / 256) .. +7, written in an order rotated by v so
    // that neighbouring lanes hit different banks
    {
        __attribute__((address_space(3))) uint64_t *lut_lds =
                (__attribute__((address_space(3))) uint64_t *)(uintptr_t)bt_lds_addr(lut_lds8);
        for (uint32_t v = threadIdx.x; v < 256u * BT_LUT_COPIES / 8u; v += blockDim.x) {
            const uint32_t b = v & 255u, c0 = 8u * (v >> 8);
            const uint2 e = bt_lut_entry(b);
            const uint64_t e64 = ((uint64_t)e.y << 32) | e.x;
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) lut_lds[b * BT_LUT_COPIES + c0 + ((k + v) & 7u)] = e64;
        }
    }

    // (5) blocks in order, one barrier each. After the barrier of block i
    // each lane can take its start from the row totals posted above, Y of
    // block i-1 is complete (every wavefront's partial is in) and staging
    // buffer (i-1) % nbuf is free for the next payload.
    // Sums rotate over three buffers: block i adds into i % 3 after barrier
    // i, block i-1's are read after barrier i, and i+1 % 3 (last read before
    // barrier i) is cleared after barrier i for block i+1.
    auto write_y = [&](int i) -> void {
        const int m0 = (b_begin + i) * BT_ROWS;
        const int rows = min(BT_ROWS, M - m0);
        const int32_t *s = sums + (i % 3) * NB * 256;
        // D layout of v_mfma_i32_16x16x64_i8: lane l, register k -> row 4*(l/16)+k, column l%16
        for (int o = threadIdx.x; o < NB * 256; o += blockDim.x) {
            const int nb = o >> 8, col = (o >> 4) & 15, rl = o & 15;
            const int ln = (rl >> 2) * 16 + col, k = rl & 3;
            const int n = col + 16 * nb;
            if (n < N && rl < rows) bt_store_y1(Y, epi, M, n, m0 + rl, s[(nb * 4 + k) * 64 + ln]);
        }
    };
    // decode + contract block i into acc (after its barrier)
    auto decode_block = [&](int i, bt_v4i (&acc)[NB]) -> void {
        const bool in_lds = fits(i);
        const BtRange g = bt_range<WB>(nib[i], nib[i + 1]);
        const int rows = min(BT_ROWS, M - (b_begin + i) * BT_ROWS);
        const int32_t *wti = wt + i * BT_ROWS * WC;
        // lane start: rows before r, wavefronts before this one, lane groups before q
        uint32_t pstart;
        {
            // prefix over the wavefronts' totals; the wave-uniform indices
            // become one indexed register read each
            uint32_t pre[WC + 1];
            pre[0] = 0;
#pragma unroll
            for (int w4 = 0; w4 < WC; w4 += 4) {
                const bt_v4i t4 = *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(wti + r * WC + w4);
                pre[w4 + 1] = pre[w4] + (uint32_t)t4.x;
                pre[w4 + 2] = pre[w4 + 1] + (uint32_t)t4.y;
                pre[w4 + 3] = pre[w4 + 2] + (uint32_t)t4.z;
                pre[w4 + 4] = pre[w4 + 3] + (uint32_t)t4.w;
            }
            const uint32_t row_total = pre[nwaves], before_w = pre[wave];
            // exclusive prefix of row totals over r inside each 16-lane DPP row
            uint32_t sc = row_total;
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x111, 0xF, 0xF, true);   // row_shr:1
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x112, 0xF, 0xF, true);   // row_shr:2
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x114, 0xF, 0xF, true);   // row_shr:4
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x118, 0xF, 0xF, true);   // row_shr:8
            // value index of the lane's first nonzero, counted from the block's first granule
            pstart = r < rows ? (nib[i] & (16u * VPB - 1u)) + (sc - row_total) + before_w + (incl[i] - seg[i]) : 0u;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = bt_v4i{0, 0, 0, 0};
        uint32_t p = pstart;
        if (in_lds) {
            // a corrupt stream stays inside the staged granules
            p = min(p, 16u * VPB * g.n - 8u * VPB);
            // VPB times the buffer's address (a multiple of 16) keeps p & 7
            const uint32_t base2 = VPB * bt_lds_addr(stage + (uint32_t)(i % (int)nbuf) * stage_bytes);
            if constexpr (STG) {
                // stream nibble pt sits 3 granules (96 nibbles) further per run of 61 before it
                const auto tmap = [=](uint32_t pt) { return pt + base2 + __umulhi(pt, BT_R61_MAG) * 96u; };
                bt_contract<NB, TPL, BtWinLds, decltype(tmap)>(words[i], p, BtWinLds{}, lut_base, xb, acc, tmap);
            } else {
                bt_contract<NB, TPL, BtWinLdsT<WB>, BtTileSame, WB>(words[i], p + base2, BtWinLdsT<WB>{}, lut_base,
                                                                   xb, acc);
            }
        } else {
            bt_contract<NB, TPL, BtWinGlobalT<WB>, BtTileSame, WB>(words[i], p, BtWinGlobalT<WB>{prs, 4u * g.g0},
                                                                  lut_base, xb, acc);
        }
    };

    if (NBLK > 1 && one_pass) {
        // every block is staged at once: one barrier for all of them, each
        // wavefront's partials to its own LDS slice, one barrier, then Y
        int32_t *part = reinterpret_cast<int32_t *>(stage + nbuf * stage_bytes);   // [nblk][nwaves][NB*256]
        bt_wait_vm(0);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
            if (i >= nblk) break;
            bt_v4i acc[NB];
            decode_block(i, acc);
            // this wavefront's partial of block i, lane-major: the 4
            // accumulators of a lane side by side (one 16-byte store)
            int32_t *pw = part + (i * nwaves + wave) * NB * 256;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                *(__attribute__((address_space(3))) bt_v4i *)(uintptr_t)bt_lds_addr(pw + nb * 256 + lane * 4) =
                        bt_v4i{acc[nb][0] >> PS, acc[nb][1] >> PS, acc[nb][2] >> PS, acc[nb][3] >> PS};
        }
        __syncthreads();
        // Y: item (block i, column block nb, lane l) sums the wavefronts'
        // partials of lane l, i.e. rows 4 (l / 16) .. +3 of column l % 16
        // (the D layout of the 16x16 MFMAs), four consecutive rows of Y
        for (int o = threadIdx.x; o < nblk * NB * 64; o += blockDim.x) {
            const int i = o / (NB * 64), nb = (o / 64) % NB, ln = o % 64;
            const int n = (ln & 15) + 16 * nb;
            const int m = (b_begin + i) * BT_ROWS + 4 * (ln >> 4);
            if (n >= N || m >= M) continue;
            bt_v4i v = {0, 0, 0, 0};
            for (int w = 0; w < nwaves; ++w)
                v += *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(part + ((i * nwaves + w) * NB + nb) * 256 + ln * 4);
            bt_store_y4(Y, epi, M, n, m, v);
        }
        return;
    }

#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
        if (i >= nblk) break;
        bt_wait_vm(vm_issued - vm_mark[i]);   // this wavefront's share of block i landed
        __syncthreads();                      // ... everyone's; block i-1 is decoded and summed
        if (i > 0) {
            write_y(i - 1);
            if (i - 1 + (int)nbuf < nblk) issue_block(i - 1 + (int)nbuf);
        }
        if (i >= 2)
            for (int o = threadIdx.x; o < NB * 256; o += blockDim.x) sums[((i + 1) % 3) * NB * 256 + o] = 0;
        bt_v4i acc[NB];
        decode_block(i, acc);
        // the wavefronts' partials (each exact after >> PS) meet in LDS
        int32_t *sp = sums + (i % 3) * NB * 256;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < 4; ++k) atomicAdd(&sp[(nb * 4 + k) * 64 + lane], acc[nb][k] >> PS);
    }
    __syncthreads();
    write_y(nblk - 1);
}

// Streaming variant for TPL = 2 (K <= 4096) and at most BTS_NBLK blocks per
// workgroup. Each wavefront issues D payload DMA instructions (1 KB each) per
// block, a fixed count, so the vector-memory counter tells exactly when block
// i has landed; granules past the block read as zeros. A block with more
// granules than the D KB per wavefront hold is decoded from global memory
// instead. One block is in flight at a time: block i + 1 (its bitmap words,
// then its payload) is issued once block i has landed, so the memory system
// delivers the blocks in order (with two or more in flight each lands later)
// and block i is decoded while the next one streams in. Per block: words ->
// row totals -> wait for its payload -> barrier -> decode into a
// per-wavefront partial slice. The barrier is an LDS-only one, so it never
// waits for the later blocks' transfers.
#define BTS_NBLK 3
#define BTS_RUN 64u              // granules per run of the staggered staging (1 KB)
#define BTS_RUN_NIB_LOG2 11      // log2 of the nibbles in a run
#define BTS_OVL 3u               // granules stored again after each run: a tile's windows reach < 48 B past its start
#define BTS_DIVMAG 15651u        // ceil(2^20 / (BTS_RUN + BTS_OVL)): exact quotient for slots < 2^14

// B operands of the lane's tiles from their X slices
template <int NB, int TPL>
__device__ __forceinline__ void bt_make_b(const uint32_t (&xw)[NB][TPL][8], bt_v4i (&xb)[NB][TPL][4]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int k = 0; k < TPL; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xb[nb][k][j] = bt_b_operand(xw[nb][k][2 * j], xw[nb][k][2 * j + 1]);
                asm volatile("" : "+v"(xb[nb][k][j]));
            }
}

// The work of one workgroup; gid is its index among the workgroups of its
// matrix (the plain kernel's block index, or its place in a grouped launch).
// WB: width of a stored weight value (4: int4; 2: int2, the W2A4 variant).
template <int NB, int D, bool XU, int NBLK = BTS_NBLK, int WB = 4>
__device__ __forceinline__ void bts_body(
        int gid, const uint32_t *__restrict__ offsets, int M, int K, int bq, int br,
        const uint64_t *__restrict__ bitmaps, const uint8_t *__restrict__ X, int N,
        const uint8_t *__restrict__ payload, uint32_t payload_bytes, int32_t *__restrict__ Y, uint32_t stagger,
        uint32_t area_kb, const BtEpi epi) {
    constexpr int TPL = 2, WC = 8;
    extern __shared__ __attribute__((aligned(16))) uint8_t bt_smem[];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int T = (K + 63) >> 6;
    const int b_begin = gid * bq + min(gid, br);
    const int nblk = bq + (gid < br ? 1 : 0);           // 1 .. NBLK
    const int t0 = (wave * 4 + q) * TPL;
    const uint32_t xs = ((uint32_t)K + 1u) >> 1;
    asm volatile("" ::"s"(bitmaps), "s"(payload), "s"(X), "s"(Y), "s"(N), "s"(payload_bytes));

    // LDS: selector table | row totals [NBLK][16][WC] | partials
    // [nblk_max][nwaves][NB*256] | staging [nblk_max][area_kb KB] | 1 KB
    // dummy; staging area i holds block i's payload, 1 KB per DMA
    // instruction, dealt round robin to the wavefronts (D each)
    const uint32_t lut_base = bt_lds_addr(bt_smem) + (uint32_t)(lane % BT_LUT_COPIES) * 8u;
    int32_t *wt = reinterpret_cast<int32_t *>(bt_smem + BT_LUT_BYTES);
    int32_t *part = wt + NBLK * BT_ROWS * WC;
    const int nblk_max = bq + (br > 0 ? 1 : 0);
    uint8_t *stage = reinterpret_cast<uint8_t *>(part + nblk_max * nwaves * NB * 256);
    const uint32_t area = area_kb * 1024u;
    // Staggered staging (stagger = 1): the stream is cut in runs of
    // BTS_RUN granules, each stored with the next BTS_OVL granules after it,
    // so every run starts BTS_OVL granules (48 B) further round the LDS banks
    // than the stream would put it. Rows whose length is close to a multiple
    // of 256 B otherwise put the same tile of every row on the same banks.
    // Granule u of the stream sits in slot u + BTS_OVL * (u / BTS_RUN); slot s
    // holds granule s - BTS_OVL * (s / (BTS_RUN + BTS_OVL)).
    const uint32_t slots = area_kb * 64u;
    const uint32_t cap = stagger ? BTS_RUN * (slots / (BTS_RUN + BTS_OVL)) : slots;   // granules a block's area holds
    const uint32_t kmag = stagger ? BTS_DIVMAG : 0u;             // s * kmag >> 20 = s / (BTS_RUN + BTS_OVL)
    constexpr uint32_t VPB = 8 / WB;                               // values per payload byte
    constexpr int PS = WB == 4 ? 8 : 10;                           // log2 of the A x B operand scale
    const uint32_t tmul = stagger ? VPB * 16u * BTS_OVL : 0u;    // values added per run
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(payload, payload_bytes);

    uint32_t nib[NBLK + 1];
#pragma unroll
    for (int i = 0; i <= NBLK; ++i) {
        const int b = b_begin + (i < nblk ? i : nblk);
        nib[i] = offsets[(int64_t)min(b * BT_ROWS, M) * T];
    }
    asm volatile("" ::: "memory");

    // X slices of the lane's tiles (zeros past N or T), loaded first; they
    // become B operands only once block 0 has landed, so that the first
    // payload DMA goes out as soon as the block offsets are in (waiting for
    // X first held it back by about half a microsecond)
    // (in runs of 16 rows at N > 16, where that gains 0.35 us on 12288 x 4096
    // at N = 32; at N <= 16 per-lane slices, 0.05 us faster there at N = 8)
    bt_v4i xg[NB][2 * TPL];
    uint32_t xw[NB][TPL][8];
    {
        const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(X, bt_x_range(N, xs));
        if constexpr (NB == 2) {
            bt_load_x_runs<NB, TPL, XU>(xrs, r, q, wave, T, N, xs, xg);
        } else {
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int n = r;
                const uint32_t off = (n < N && t0 + k < T) ? (uint32_t)n * xs + (uint32_t)(t0 + k) * 32u : 0xFFFFFFE0u;
                const bt_v4i v0 = bt_load_x16<XU>(xrs, off);
                const bt_v4i v1 = bt_load_x16<XU>(xrs, off + 16u);
                xw[0][k][0] = v0.x; xw[0][k][1] = v0.y; xw[0][k][2] = v0.z; xw[0][k][3] = v0.w;
                xw[0][k][4] = v1.x; xw[0][k][5] = v1.y; xw[0][k][6] = v1.z; xw[0][k][7] = v1.w;
            }
        }
    }
    // bitmap words: block 0's now, block i + 1's with its DMA (below), so
    // that the first payload does not queue behind every block's words (a
    // row past M or past the workgroup's range is past the end of the buffer
    // and reads zeros; a tile past the row's end is cleared before use)
    const int m_first = b_begin * BT_ROWS;
    const int wg_rows = min(nblk * BT_ROWS, M - m_first);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(bitmaps + (int64_t)m_first * T, (uint32_t)wg_rows * (uint32_t)T * 8u);
    uint64_t words[NBLK][TPL];
    auto load_words = [&](int i) -> void {
        const int rr = i * BT_ROWS + r;
        const uint32_t off = ((uint32_t)rr * (uint32_t)T + (uint32_t)t0) * 8u;
        const bt_v4i v = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, BT_NT));
        words[i][0] = ((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x;
        words[i][1] = ((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z;
    };
    load_words(0);
    bt_v4i xb[NB][TPL][4];   // B operands, made from xw once block 0 has landed
    // payload of block i < nblk: every wavefront issues exactly D
    // instructions per block, also for KB past the area, which write zeros
    // into a 1 KB dummy slot behind the staging areas. With a fixed count in straight-line code the compiler's
    // own waits are exact (block 0's words are used before its payload has
    // landed); with a count that depends on the wavefront it waits for
    // everything in flight.
    uint8_t *dummy = stage + (uint32_t)nblk_max * area;
    auto issue = [&](int i) -> void {
        const bool blk = i < nblk;
        const BtRange g = bt_range<WB>(nib[i], nib[i + 1]);
        const uint32_t n = blk ? min(g.n, cap) : 0u;
        uint8_t *buf = stage + (uint32_t)i * area;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const uint32_t j = (uint32_t)(wave + nwaves * d);
            const bool real = blk && j < area_kb;   // wave-uniform
            const uint32_t sl = j * 64u + (uint32_t)lane;
            const uint32_t u = sl - BTS_OVL * ((sl * kmag) >> 20);   // stream granule of slot sl
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(real ? buf + j * 1024u : dummy), 16,
                                                     (real && u < n) ? (g.g0 + u) * 16u : 0xFFFFFFF0u, 0, 0, BT_NT);
        }
    };
    // one block in flight: the memory system serves it before any later
    // block, which is issued only once block i has landed
    issue(0);
    {
        __attribute__((address_space(3))) uint64_t *lut_lds =
                (__attribute__((address_space(3))) uint64_t *)(uintptr_t)bt_lds_addr(bt_smem);
        for (uint32_t v = threadIdx.x; v < 256u * BT_LUT_COPIES / 8u; v += blockDim.x) {
            const uint32_t b = v & 255u, c0 = 8u * (v >> 8);
            const uint2 e = bt_lut_entry(b);
            const uint64_t e64 = ((uint64_t)e.y << 32) | e.x;
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) lut_lds[b * BT_LUT_COPIES + c0 + ((k + v) & 7u)] = e64;
        }
    }

#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
        if (i >= nblk) break;
        // words of block i -> segment popcounts, lane-group prefix, row totals
#pragma unroll
        for (int k = 0; k < TPL; ++k)
            if (t0 + k >= T) words[i][k] = 0;
        uint32_t seg = 0;
#pragma unroll
        for (int k = 0; k < TPL; ++k) seg += (uint32_t)__builtin_popcountll(words[i][k]);
        uint32_t incl = seg;
        {
            const uint32_t u16 = (uint32_t)__shfl_up((int)incl, 16, 64);
            incl += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)incl, 32, 64);
            incl += q >= 2 ? u32 : 0u;
        }
        int32_t *wti = wt + i * BT_ROWS * WC;
        if (q == 3) wti[r * WC + wave] = (int32_t)incl;
        bt_wait_vm(0);   // this wavefront's share of block i landed (nothing later is in flight)
        if (i + 1 < nblk) {
            load_words(i + 1);   // ahead of its payload: block i + 1's row totals need no wait for it
            issue(i + 1);
        }
        if (i == 0) {
            // X landed with block 0 (waited above)
            if constexpr (NB == 2) bt_x_runs_to_slices<NB, TPL>(xg, xw);
            bt_make_b<NB, TPL>(xw, xb);
        }
        bt_barrier_lds();                     // ... everyone's, and every row total of block i
        const BtRange g = bt_range<WB>(nib[i], nib[i + 1]);
        const int rows = min(BT_ROWS, M - (b_begin + i) * BT_ROWS);
        uint32_t pstart;
        {
            // prefix over the wavefronts' totals; the wave-uniform indices
            // become one indexed register read each
            uint32_t pre[WC + 1];
            pre[0] = 0;
#pragma unroll
            for (int w4 = 0; w4 < WC; w4 += 4) {
                const bt_v4i t4 = *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(wti + r * WC + w4);
                pre[w4 + 1] = pre[w4] + (uint32_t)t4.x;
                pre[w4 + 2] = pre[w4 + 1] + (uint32_t)t4.y;
                pre[w4 + 3] = pre[w4 + 2] + (uint32_t)t4.z;
                pre[w4 + 4] = pre[w4 + 3] + (uint32_t)t4.w;
            }
            const uint32_t row_total = pre[nwaves], before_w = pre[wave];
            uint32_t sc = row_total;
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x111, 0xF, 0xF, true);   // row_shr:1
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x112, 0xF, 0xF, true);   // row_shr:2
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x114, 0xF, 0xF, true);   // row_shr:4
            sc += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sc, 0x118, 0xF, 0xF, true);   // row_shr:8
            pstart = r < rows ? (nib[i] & (16u * VPB - 1u)) + (sc - row_total) + before_w + (incl - seg) : 0u;
        }
        bt_v4i acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = bt_v4i{0, 0, 0, 0};
        if (g.n <= cap) {
            // a corrupt stream stays inside the staged granules
            // (a tile's windows stay inside the run of its first nonzero plus
            // the BTS_OVL granules stored after it)
            const uint32_t p = min(pstart, 16u * VPB * g.n - 8u * VPB);
            const uint32_t base2 = VPB * bt_lds_addr(stage + (uint32_t)i * area);
            const auto tmap = [=](uint32_t pt) { return pt + base2 + (pt >> (BTS_RUN_NIB_LOG2 + (WB == 2))) * tmul; };
            bt_contract<NB, TPL, BtWinLdsT<WB>, decltype(tmap), WB>(words[i], p, BtWinLdsT<WB>{}, lut_base, xb, acc,
                                                                    tmap);
        } else {
            bt_contract<NB, TPL, BtWinGlobalT<WB>, BtTileSame, WB>(words[i], pstart, BtWinGlobalT<WB>{prs, 4u * g.g0},
                                                                  lut_base, xb, acc);
        }
        int32_t *pw = part + (i * nwaves + wave) * NB * 256;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *(__attribute__((address_space(3))) bt_v4i *)(uintptr_t)bt_lds_addr(pw + nb * 256 + lane * 4) =
                    bt_v4i{acc[nb][0] >> PS, acc[nb][1] >> PS, acc[nb][2] >> PS, acc[nb][3] >> PS};
    }
    bt_barrier_lds();
    // Y: item (block i, column block nb, lane l) sums the wavefronts' partials
    // of lane l: rows 4 (l / 16) .. +3 of column l % 16 (the MFMA D layout)
    for (int o = threadIdx.x; o < nblk * NB * 64; o += blockDim.x) {
        const int i = o / (NB * 64), nb = (o / 64) % NB, ln = o % 64;
        const int n = (ln & 15) + 16 * nb;
        const int m = (b_begin + i) * BT_ROWS + 4 * (ln >> 4);
        if (n >= N || m >= M) continue;
        bt_v4i s = bt_v4i{0, 0, 0, 0};
        for (int w = 0; w < nwaves; ++w)
            s += *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(part + ((i * nwaves + w) * NB + nb) * 256 + ln * 4);
        bt_store_y4(Y, epi, M, n, m, s);
    }
}

template <int NB, int D, bool XU>
__global__ __launch_bounds__(512) void k_bt64s_w4a4(
        const uint32_t *__restrict__ offsets, int M, int K, int bq, int br, const uint64_t *__restrict__ bitmaps,
        const uint8_t *__restrict__ X, int N, const uint8_t *__restrict__ payload, uint32_t payload_bytes,
        int32_t *__restrict__ Y, uint32_t stagger, uint32_t area_kb, uint16_t *Yh, const float *sw, const float *sx) {
    bts_body<NB, D, XU>((int)blockIdx.x, offsets, M, K, bq, br, bitmaps, X, N, payload, payload_bytes, Y, stagger,
                        area_kb, BtEpi{Yh, sw, sx});
}

// W2A4: 2-bit weights (UnionSparse Sec. VII, Fig. 11) through the same
// streaming kernel; int32 Y.
template <int NB, int D, bool XU>
__global__ __launch_bounds__(512) void k_bt64s_w2a4(
        const uint32_t *__restrict__ offsets, int M, int K, int bq, int br, const uint64_t *__restrict__ bitmaps,
        const uint8_t *__restrict__ X, int N, const uint8_t *__restrict__ payload, uint32_t payload_bytes,
        int32_t *__restrict__ Y, uint32_t stagger, uint32_t area_kb) {
    bts_body<NB, D, XU, BTS_NBLK, 2>((int)blockIdx.x, offsets, M, K, bq, br, bitmaps, X, N, payload, payload_bytes, Y,
                                     stagger, area_kb, BtEpi{nullptr, nullptr, nullptr});
}

// Grouped launch: up to BTS_GROUP_MAX matrices with one K, each with its own
// stream, X, output and epilogue, in one dispatch; item i owns the
// workgroups [wg_begin, next item's wg_begin). A workgroup takes up to
// BTS_GROUP_NBLK blocks, one more than the plain kernel: items whose blocks
// do not divide evenly into the CUs then fit in one round of workgroups.
#define BTS_GROUP_MAX 8
#define BTS_GROUP_NBLK 4
struct BtsItem {
    const uint32_t *offsets;
    const uint64_t *bitmaps;
    const uint8_t *X;
    const uint8_t *payload;
    int32_t *Y;
    uint16_t *Yh;
    const float *sw;
    const float *sx;
    int M, N, bq, br, wg_begin;
    uint32_t payload_bytes, stagger, area_kb;
};
struct BtsGroup {
    int count, K;
    BtsItem item[BTS_GROUP_MAX];
};

template <int NB, int D, bool XU>
__global__ __launch_bounds__(512) void k_bt64s_group(const BtsGroup g) {
    const int wg = (int)blockIdx.x;
    // the item of this workgroup (uniform; every field read at a fixed offset)
    BtsItem it = g.item[0];
#pragma unroll
    for (int j = 1; j < BTS_GROUP_MAX; ++j)
        if (j < g.count && wg >= g.item[j].wg_begin) it = g.item[j];
    bts_body<NB, D, XU, BTS_GROUP_NBLK>(wg - it.wg_begin, it.offsets, it.M, g.K, it.bq, it.br, it.bitmaps, it.X, it.N,
                                        it.payload, it.payload_bytes, it.Y, it.stagger, it.area_kb,
                                        BtEpi{it.Yh, it.sw, it.sx});
}

// LDS of the streaming variant: the selector table, the row totals, for each
// of a workgroup's nblk blocks the wavefronts' partials and area_kb KB of
// staging, and the 1 KB dummy slot of the unused DMA instructions
static size_t bts_lds(int nwaves, int nb, int64_t area_kb, int64_t nblk, int nblk_cap = BTS_NBLK) {
    return (size_t)BT_LUT_BYTES + (size_t)nblk_cap * BT_ROWS * 8 * 4 +
           (size_t)nblk * ((size_t)nwaves * nb * 256 * 4 + (size_t)area_kb * 1024) + 1024;
}

// Launch plan.
struct BtPlan {
    int nwaves, nb, tpl;
    unsigned grid;
    int bq, br;             // blocks per workgroup: bq, plus one for the first br workgroups
    uint32_t stage_bytes;   // one staging buffer
    uint32_t nbuf;          // staging buffers in the ring
    int streaming;          // > 0: the streaming variant k_bt64s_w4a4, at most this many DMA instructions per wavefront and block
    int stagger;            // staggered staging (rows near a multiple of 256 B, ring kernel 64 B, long)
    int area_kb;            // streaming variant: KB of staging per block
    int one_pass;           // every block staged at once: one barrier before and one after the decode
    int nblk;               // ring kernel: blocks per workgroup, at most (a template argument)
    size_t lds;             // total dynamic LDS
};

// Fast-path constraints: K within 8 wavefronts x 4 lane groups x 8 tiles
// (K <= 16384), N <= 32. Any K % 64: the tail of the last tile has zero bits,
// and X rows off a 4-byte boundary take the funnel-shifted loads.
static bool bt64_supported(int64_t K, int64_t N) {
    return K > 0 && (K + 63) / 64 <= 8 * 4 * 8 && N >= 1 && N <= 32;
}

static bool bt64_plan(int64_t M, int64_t K, int64_t N, int64_t payload_bytes, BtPlan *p, int wb = 4) {
    if (!bt64_supported(K, N) || M <= 0) return false;
    const int64_t T = (K + 63) / 64;
    p->tpl = T <= 64 ? 2 : T <= 128 ? 4 : 8;
    p->nwaves = (int)((T + 4 * p->tpl - 1) / (4 * p->tpl));
    p->nb = N <= 16 ? 1 : 2;
    const int64_t blocks = (M + BT_ROWS - 1) / BT_ROWS;
    // at 2 tiles per lane up to 8 blocks per workgroup where 4 would need
    // more than one workgroup per CU (rounds): int4 at N = 8, density 0.5,
    // 20000 x 4096 took 22.1 us in 1.22 rounds of 4, 16384 rows 12.6
    int64_t nblk_max = BT_NBLK(p->tpl);
    if (p->tpl == 2 && blocks > BT_CUS * nblk_max && blocks <= BT_CUS * 8) nblk_max = 8;
    if (p->tpl == 4 && p->nb == 1 && blocks > BT_CUS * nblk_max && blocks <= BT_CUS * 4) nblk_max = 4;
    p->nblk = (int)nblk_max;
    // one workgroup per CU when that leaves each at most nblk_max blocks
    const int64_t grid0 = std::max<int64_t>(std::min<int64_t>(blocks, BT_CUS), (blocks + nblk_max - 1) / nblk_max);
    const int64_t per_wg0 = (blocks + grid0 - 1) / grid0;                 // blocks of the busiest workgroup
    const int64_t wg_per_cu = (grid0 + BT_CUS - 1) / BT_CUS;
    // Staging: 1.2x the average block plus 2 KB (a denser block falls back
    // to global-memory windows), capped at the densest block; staggered, in
    // whole runs of 61 granules per KB.
    const int64_t avg = payload_bytes / std::max<int64_t>(blocks, 1);
    const int64_t worst = (int64_t)BT_ROWS * T * 8 * wb + 64;   // a fully dense block
    const int64_t est = std::min<int64_t>(worst, avg + avg / 5 + 2048) + 32;
    const int64_t fixed = BT_LUT_BYTES + nblk_max * BT_ROWS * (BT_WG_THREADS(p->tpl) / 64) * 4 + 3 * p->nb * 256 * 4;
    struct Fit {
        int64_t stage, grid, per_wg, budget, nbuf, one_pass;
    };
    // A buffer is refilled one block after it was decoded, so a ring of one
    // works only when it never refills. When the workgroups sharing a CU
    // leave too little for two buffers, size for one resident workgroup per
    // CU (the grid then runs in rounds; int4 at N = 8: 8192 x 16384 51.6 ->
    // 25.1 us, 16384 x 8192 31.1 -> 21.8, 65536 x 4096 48.3 -> 42.6); when
    // that is still short, one block per workgroup (8192 x 8192 at density
    // 0.9: 24.8 -> 15.7 us). nbuf = 0: the blocks are too dense to stage.
    const auto fit = [&](bool stg) -> Fit {
        Fit f{(stg ? (est / 16 + BT_R61_RUN) / BT_R61_RUN : (est + 1023) / 1024) * 1024, grid0, per_wg0,
              BT_LDS_MAX / wg_per_cu, 0};
        f.nbuf = std::min((f.budget - fixed) / f.stage, f.per_wg);
        if (f.nbuf < std::min<int64_t>(2, f.per_wg) && wg_per_cu > 1) {
            f.budget = BT_LDS_MAX;
            f.nbuf = std::min((f.budget - fixed) / f.stage, f.per_wg);
        }
        if (f.nbuf < std::min<int64_t>(2, f.per_wg) && f.per_wg > 1 && fixed + f.stage <= BT_LDS_MAX) {
            f.grid = blocks;
            f.per_wg = 1;
            f.budget = BT_LDS_MAX;
            f.nbuf = 1;
        }
        if (f.nbuf < std::min<int64_t>(2, f.per_wg)) f.nbuf = 0;
        // all of a workgroup's blocks staged at once, with room for
        // per-wavefront partials: decode without a barrier between blocks
        const int64_t st = f.nbuf ? f.stage : 0, nb = std::max<int64_t>(f.nbuf, 1);
        f.one_pass = nblk_max > 1 && (st == 0 || nb >= f.per_wg) &&
                     fixed + nb * st + f.per_wg * p->nwaves * p->nb * 256 * 4 <= f.budget;
        return f;
    };
    // Staggered when the average row is within 12 B of a multiple of 64 B
    // and the staggered buffers hold as many blocks as the plain ones, in
    // the same number of passes (rows of one length, int4 at N = 8: 4096 x
    // 14336 14.75 -> 12.16 us, 4096 x 11008 at N = 16 12.34 -> 11.38,
    // 5120 x 5120 10.11 -> 9.39; iid masks 4096 x 16384 13.97 -> 13.04,
    // 4096 x 11008 11.39 / 11.47). An average row of exactly such a length
    // (every row dense, or cut to one count) takes it even at the cost of
    // the single pass (12288 x 4096 dense: 18.75 -> 13.10 us).
    const int64_t rb64 = (payload_bytes / std::max<int64_t>(M, 1)) % 64;
    Fit f = fit(false);
    p->stagger = 0;
    if (wb == 4 && std::min<int64_t>(rb64, 64 - rb64) < 12 && f.nbuf > 0) {
        const Fit fs = fit(true);
        if (fs.nbuf == f.nbuf && fs.grid == f.grid && (fs.one_pass == f.one_pass || rb64 == 0)) {
            f = fs;
            p->stagger = 1;
        }
    }
    int64_t stage = f.stage, nbuf = f.nbuf;
    const int64_t per_wg = f.per_wg, budget = f.budget;
    p->grid = (unsigned)f.grid;
    p->bq = (int)(blocks / f.grid);
    p->br = (int)(blocks % f.grid);
    if (nbuf == 0) {
        // blocks too dense to stage: every block reads its windows from
        // global memory (a zero-byte staging buffer fits no block)
        stage = 0;
        nbuf = 1;
    }
    const int64_t part = per_wg * p->nwaves * p->nb * 256 * 4;
    p->one_pass = (int)f.one_pass;
    p->stage_bytes = (uint32_t)stage;
    p->nbuf = (uint32_t)nbuf;
    p->lds = (size_t)(fixed + nbuf * stage + (p->one_pass ? part : 0));
    // streaming variant: D KB per wavefront and block covers the same
    // estimate as the staging buffer above
    p->streaming = 0;
    if (p->tpl == 2) {
        // staging per block: the estimate above in whole KB (with 3 extra
        // granules per 64 when staggered), at least 2 KB per wavefront
        // average payload bytes per row within 28 B of a multiple of 256 or
        // 12 B of a multiple of 128: the same tile of every row, or of every
        // other row, falls on the same LDS banks when the rows are of one
        // length (12288 x 4096 at N = 8, rows of 1152 B: 10.45 -> 9.13 us;
        // iid masks of that density 9.11 / 9.28). Elsewhere the plain layout
        // does as well or better (within 28 B of a multiple of 128 as well:
        // 12288 x 4096 at density 0.3 8.16 -> 8.67 us; 4096 x 4096 at 0.95,
        // whose blocks above the average then overflow the staggered area,
        // 5.55 -> 7.47)
        const int64_t rpb = payload_bytes / std::max<int64_t>(M, 1), rb = rpb % 256, rb2 = rpb % 128;
        int stagger = std::min<int64_t>(rb, 256 - rb) < 28 || std::min<int64_t>(rb2, 128 - rb2) < 12;
        const int64_t need = (stagger ? est * (BTS_RUN + BTS_OVL) / BTS_RUN : est) + 1023;
        const int64_t area_kb = std::min<int64_t>(4 * p->nwaves, std::max<int64_t>(2 * p->nwaves, need / 1024));
        const int d = (int)((area_kb + p->nwaves - 1) / p->nwaves);   // DMA instructions per wavefront at most
        // bytes an area holds; when the average block (plus its window
        // granule) does not fit the staggered layout the plain one is taken,
        // and when it fits neither, most blocks would read their windows from
        // global memory: the ring kernel stages them instead (12288 x 4096
        // at density 0.99: 16.2 us streaming, 11.4 in the ring kernel)
        if (stagger && avg + 64 > area_kb * 1024 * BTS_RUN / (BTS_RUN + BTS_OVL)) stagger = 0;
        const bool avg_fits = avg + 64 <= area_kb * 1024;
        if (per_wg <= BTS_NBLK && avg_fits && (int64_t)bts_lds(p->nwaves, p->nb, area_kb, per_wg) <= budget) {
            p->streaming = d;
            p->area_kb = (int)area_kb;
            p->stagger = stagger;
            p->lds = bts_lds(p->nwaves, p->nb, area_kb, per_wg);
        }
    }
    return true;
}

template <int NB, int TPL, bool XU, bool STG, int WB, int NBLK>
static void launch_bt64_n(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                          const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                          int32_t *Y, const BtEpi &e, hipStream_t stream) {
    (void)hipFuncSetAttribute((const void *)k_bt64_w4a4<NB, TPL, XU, STG, WB, NBLK>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    hipLaunchKernelGGL((k_bt64_w4a4<NB, TPL, XU, STG, WB, NBLK>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream,
                       offsets, M, K, p.bq, p.br, bitmaps, X, N, payload, payload_bytes, Y, p.stage_bytes, p.nbuf,
                       p.one_pass, e.Yh, e.sw, e.sx);
}

template <int NB, int TPL, bool XU, bool STG, int WB = 4>
static void launch_bt64_s(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                          const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                          int32_t *Y, const BtEpi &e, hipStream_t stream) {
    if constexpr (TPL == 2) {
        if (p.nblk == 8) {
            launch_bt64_n<NB, TPL, XU, STG, WB, 8>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e,
                                                   stream);
            return;
        }
    }
    if constexpr (TPL == 4 && NB == 1) {   // (two column blocks would spill)
        if (p.nblk == 4) {
            launch_bt64_n<NB, TPL, XU, STG, WB, 4>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e,
                                                   stream);
            return;
        }
    }
    launch_bt64_n<NB, TPL, XU, STG, WB, BT_NBLK(TPL)>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e,
                                                      stream);
}

// W2A4 through the ring kernel (K past the streaming kernel's 4096), int32 Y
// (the plan is bt64_plan's with 2-bit values, never staggered)
static void launch_bt64_w2a4(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                             const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                             int32_t *Y, hipStream_t stream) {
    const BtEpi e{nullptr, nullptr, nullptr};
#define BT2_LAUNCH(NB, TPL, XU) \
    launch_bt64_s<NB, TPL, XU, false, 2>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream)
#define BT2_LAUNCH_X(NB, TPL)              \
    do {                                   \
        if (K % 8 == 0)                    \
            BT2_LAUNCH(NB, TPL, false);    \
        else                               \
            BT2_LAUNCH(NB, TPL, true);     \
    } while (0)
    if (p.nb == 1) {
        if (p.tpl == 2) BT2_LAUNCH_X(1, 2); else if (p.tpl == 4) BT2_LAUNCH_X(1, 4); else BT2_LAUNCH_X(1, 8);
    } else {
        if (p.tpl == 2) BT2_LAUNCH_X(2, 2); else if (p.tpl == 4) BT2_LAUNCH_X(2, 4); else BT2_LAUNCH_X(2, 8);
    }
#undef BT2_LAUNCH_X
#undef BT2_LAUNCH
}

template <int NB, int TPL, bool XU>
static void launch_bt64_t(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                          const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                          int32_t *Y, const BtEpi &e, hipStream_t stream) {
    if (p.stagger)
        launch_bt64_s<NB, TPL, XU, true>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream);
    else
        launch_bt64_s<NB, TPL, XU, false>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream);
}

template <bool XU>
static void launch_bt64_w4a4_x(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                               const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                               int32_t *Y, const BtEpi &e, hipStream_t stream) {
    if (p.streaming) {
#define BTS_LAUNCH(NB, D)                                                                                             \
    do {                                                                                                              \
        (void)hipFuncSetAttribute((const void *)k_bt64s_w4a4<NB, D, XU>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                  (int)p.lds);                                                                        \
        hipLaunchKernelGGL((k_bt64s_w4a4<NB, D, XU>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream, offsets, M, K, \
                           p.bq, p.br, bitmaps, X, N, payload, payload_bytes, Y, (uint32_t)p.stagger,                 \
                           (uint32_t)p.area_kb, e.Yh, e.sw, e.sx);                                                    \
    } while (0)
        if (p.nb == 1) {
            if (p.streaming == 2) BTS_LAUNCH(1, 2); else if (p.streaming == 3) BTS_LAUNCH(1, 3); else BTS_LAUNCH(1, 4);
        } else {
            if (p.streaming == 2) BTS_LAUNCH(2, 2); else if (p.streaming == 3) BTS_LAUNCH(2, 3); else BTS_LAUNCH(2, 4);
        }
#undef BTS_LAUNCH
        return;
    }
#define BT_LAUNCH(NB, TPL) launch_bt64_t<NB, TPL, XU>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream)
    if (p.nb == 1) {
        if (p.tpl == 2) BT_LAUNCH(1, 2); else if (p.tpl == 4) BT_LAUNCH(1, 4); else BT_LAUNCH(1, 8);
    } else {
        if (p.tpl == 2) BT_LAUNCH(2, 2); else if (p.tpl == 4) BT_LAUNCH(2, 4); else BT_LAUNCH(2, 8);
    }
#undef BT_LAUNCH
}

// X rows of ceil(K/2) bytes sit on a 4-byte boundary when K % 8 == 0
static void launch_bt64_w4a4(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                             const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                             int32_t *Y, hipStream_t stream, const BtEpi &e = BtEpi{nullptr, nullptr, nullptr}) {
    if (K % 8 == 0)
        launch_bt64_w4a4_x<false>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream);
    else
        launch_bt64_w4a4_x<true>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, e, stream);
}

// W2A4 through the streaming kernel (the plan must be a streaming one).
template <bool XU>
static void launch_bt64s_w2a4_x(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                                const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                                int32_t *Y, hipStream_t stream) {
#define BTS2_LAUNCH(NB, D)                                                                                            \
    do {                                                                                                              \
        (void)hipFuncSetAttribute((const void *)k_bt64s_w2a4<NB, D, XU>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                  (int)p.lds);                                                                        \
        hipLaunchKernelGGL((k_bt64s_w2a4<NB, D, XU>), dim3(p.grid), dim3(64 * p.nwaves), p.lds, stream, offsets, M, K, \
                           p.bq, p.br, bitmaps, X, N, payload, payload_bytes, Y, (uint32_t)p.stagger,                 \
                           (uint32_t)p.area_kb);                                                                      \
    } while (0)
    if (p.nb == 1) {
        if (p.streaming == 2) BTS2_LAUNCH(1, 2); else if (p.streaming == 3) BTS2_LAUNCH(1, 3); else BTS2_LAUNCH(1, 4);
    } else {
        if (p.streaming == 2) BTS2_LAUNCH(2, 2); else if (p.streaming == 3) BTS2_LAUNCH(2, 3); else BTS2_LAUNCH(2, 4);
    }
#undef BTS2_LAUNCH
}

static void launch_bt64s_w2a4(const BtPlan &p, const uint64_t *bitmaps, const uint32_t *offsets,
                              const uint8_t *payload, uint32_t payload_bytes, int M, int K, const uint8_t *X, int N,
                              int32_t *Y, hipStream_t stream) {
    if (K % 8 == 0)
        launch_bt64s_w2a4_x<false>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, stream);
    else
        launch_bt64s_w2a4_x<true>(p, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y, stream);
}

// Grouped launch of the streaming kernel (items prepared by the caller:
// plans with one nwaves, NB the widest item's, D the largest).
template <bool XU>
static void launch_bts_group_x(const BtsGroup &g, int nb, int d, unsigned grid, int nwaves, size_t lds,
                               hipStream_t stream) {
#define BTG_LAUNCH(NB, D)                                                                                             \
    do {                                                                                                              \
        (void)hipFuncSetAttribute((const void *)k_bt64s_group<NB, D, XU>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                  (int)lds);                                                                          \
        hipLaunchKernelGGL((k_bt64s_group<NB, D, XU>), dim3(grid), dim3(64 * nwaves), lds, stream, g);                \
    } while (0)
    if (nb == 1) {
        if (d == 2) BTG_LAUNCH(1, 2); else if (d == 3) BTG_LAUNCH(1, 3); else BTG_LAUNCH(1, 4);
    } else {
        if (d == 2) BTG_LAUNCH(2, 2); else if (d == 3) BTG_LAUNCH(2, 3); else BTG_LAUNCH(2, 4);
    }
#undef BTG_LAUNCH
}
