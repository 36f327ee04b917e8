// kernels_splitk.hip -- the bitmap SpMM over K ranges: a workgroup owns a set
// of 16-row blocks and a range of tiles of K, and the ranges of one block set
// can be spread over several workgroups whose partial sums meet in a caller
// workspace. Included after kernels_bt64.hip and kernels_bt64_f16.hip, whose
// decode and contraction helpers it uses.
//
// Why. A workgroup that owns whole rows reads all of X for them: at large
// N x K (a 4096 x 11008 down projection at N = 16, or fp16 at N = 32) X is
// most of what every CU reads. Owning 2 or 4 blocks over 1/2 or 1/4 of K
// halves or quarters the X a CU reads for the same number of weights. It
// also gives fp16 a fast path past K = 4096, where one tile per lane over all
// of K no longer fits a workgroup. The split follows the pages' SpMM (the
// STORETILE / REDUCTION steps of UnionSparse, Sec. VI-C, Alg. 2); the bounded
// choice of split count follows the N:M co-design page's split-K rule (a few
// candidates, chosen by shape, Sec. 4.3).
//
// Work item (set, split): blocks set * nbs .. + nbs - 1, tiles [ts, te) of K,
// walked in chunks of at most CT tiles (CT = 8 x wavefronts for int4, two
// tiles per lane; 4 x wavefronts for fp16, one tile per lane). Per chunk:
//   - row segments: the chunk's part of a row is one contiguous run of the
//     stream, [offsets[row T + cs], offsets[row T + ce]) (the format's own
//     offsets; the end of a row's last tile is the start of the next row);
//   - each segment goes to its own LDS slot by DMA, one instruction per
//     1 KB of the segment (every instruction reads one contiguous run), the
//     instructions dealt round robin to the wavefronts; slots are 64 bytes
//     longer than their instructions so consecutive rows start on different
//     LDS banks;
//   - one barrier (the DMAs landed, every wavefront's row totals posted),
//     then each lane decodes and contracts its tiles as in the other kernels,
//     its start being the segment start plus the popcounts of the tiles
//     before its own in the chunk;
//   - a second barrier before the next chunk's DMAs reuse the slots.
// A block whose segments do not all fit their slots reads its windows from
// global memory instead (decided per block, so the wavefront stays uniform).
//
// Sums. Accumulators stay in registers across the chunks. At the end the
// wavefronts' partials meet in LDS (added in wavefront order) and then
//   - one split per set: written to Y;
//   - several: written to the workspace (int32, or fp32 for fp16), and the
//     last workgroup of the set to arrive (an atomic counter per set) adds
//     the splits' partials in split order, writes Y and resets the counter
//     to zero for the next call. The result does not depend on timing.

#define SK_NBS_MAX 4             // blocks per set, at most
#define SK_SLOT_SKEW 64u         // LDS bytes added to every segment slot (bank spread)

struct SkArgs {
    const uint64_t *bitmaps;
    const uint32_t *offsets;
    const void *payload;
    uint32_t payload_bytes;
    int M, K, N, T;
    const void *X;
    void *Y;
    int nbs;            // blocks per set
    int nsets;
    int S;              // splits per set (workgroups per set)
    int tps;            // tiles per split (the last split may hold fewer)
    int iseg;           // DMA instructions (KB) per segment slot
    void *ws_part;      // S > 1: [nsets * nbs][S][N][16] partial sums (int32 or fp32)
    uint32_t *ws_cnt;   // S > 1: [nsets] arrival counters, zero between calls
};

// Row segment of row `rr` of the set (row b0 16 + rr of the matrix) over
// tiles [cs, ce): element range [a, b). ors covers the set's offsets, from
// its first row's tile 0 on. Rows past M are empty.
__device__ __forceinline__ uint2 sk_segment(__amdgpu_buffer_rsrc_t ors, int rr, bool in_m, int T, int cs, int ce) {
    if (!in_m) return uint2{0u, 0u};
    const uint32_t a = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ors, ((uint32_t)rr * (uint32_t)T + (uint32_t)cs) * 4u, 0, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ors, ((uint32_t)rr * (uint32_t)T + (uint32_t)ce) * 4u, 0, 0);
    return uint2{a, b};
}

// The set's and split's place, and the final sum (shared by both dtypes).
struct SkPlace {
    int set, split, b0, nb_here, ts, te;
};
__device__ __forceinline__ SkPlace sk_place(const SkArgs &a) {
    SkPlace p;
    p.set = (int)blockIdx.x / a.S;
    p.split = (int)blockIdx.x - p.set * a.S;
    p.b0 = p.set * a.nbs;
    const int nblocks = (a.M + 15) >> 4;
    p.nb_here = min(a.nbs, nblocks - p.b0);
    p.ts = p.split * a.tps;
    p.te = min(a.T, p.ts + a.tps);
    return p;
}

// Workspace partials are written and read with agent-scope stores and loads
// (they go to the coherence point shared by every XCD, not to this XCD's L2
// only), so a workgroup's partials are visible to the others once its stores
// have completed: no cache-wide write-back (a device fence) is needed.
template <class V>
__device__ __forceinline__ void sk_ws_store(V *p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ __forceinline__ V sk_ws_load(const V *p) {
    return __hip_atomic_load(const_cast<V *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether this workgroup is the last of its set to post its partials (S > 1);
// every thread returns the same answer. Each thread's partial stores are
// issued before the call; they complete (s_waitcnt) before the barrier, and
// the one counter increment follows the barrier, so a workgroup that sees
// the count S - 1 sees every split's partials.
__device__ __forceinline__ bool sk_last_arrival(const SkArgs &a, const SkPlace &pl, int *flag_lds) {
    __builtin_amdgcn_s_waitcnt(0);        // this thread's partial stores completed
    __syncthreads();
    if (threadIdx.x == 0)
        *flag_lds = (int)__hip_atomic_fetch_add(&a.ws_cnt[pl.set], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *flag_lds == a.S - 1;
}

// The counter back to zero for the next call (the last arrival only).
__device__ __forceinline__ void sk_reset(const SkArgs &a, const SkPlace &pl) {
    if (threadIdx.x == 0) sk_ws_store(&a.ws_cnt[pl.set], 0u);
}

// ------------------------------------------------------------------ int4

template <int NB, bool XU>
__global__ __launch_bounds__(512) void k_bsk_w4a4(SkArgs a) {
    constexpr int TPL = 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t sk_smem[];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int M = a.M, T = a.T, N = a.N;
    const int CT = 8 * nwaves;                                   // tiles per chunk
    const SkPlace pl = sk_place(a);
    const uint32_t xs = ((uint32_t)a.K + 1u) >> 1;
    const uint32_t slot_bytes = (uint32_t)a.iseg * 1024u + SK_SLOT_SKEW;

    // LDS: selector table (as in the other int4 kernels) | row totals
    // [NBS_MAX][16][nwaves] | segment slots [nbs][16] (after the last chunk:
    // the wavefronts' partials [nbs][nwaves][NB * 256], which fit them) | flag
    const uint32_t lut_base = bt_lds_addr(sk_smem) + (uint32_t)(lane % BT_LUT_COPIES) * 8u;
    int32_t *wt = reinterpret_cast<int32_t *>(sk_smem + BT_LUT_BYTES);
    uint8_t *slots = reinterpret_cast<uint8_t *>(wt + SK_NBS_MAX * 16 * nwaves);
    int32_t *part = reinterpret_cast<int32_t *>(slots);
    int *flag = reinterpret_cast<int *>(slots + (uint32_t)a.nbs * 16u * slot_bytes);

    // the set's rows of words and offsets (rows past M are past the range)
    const int set_rows = min(pl.nb_here * 16, M - pl.b0 * 16);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(a.payload, a.payload_bytes);
    const __amdgpu_buffer_rsrc_t ors = bt_rsrc(a.offsets + (int64_t)pl.b0 * 16 * T, ((uint32_t)set_rows * (uint32_t)T + 1u) * 4u);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(a.bitmaps + (int64_t)pl.b0 * 16 * T, (uint32_t)set_rows * (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(a.X, bt_x_range(N, xs));

    // the selector table's copies (entry b of copy c at slot 16 b + c)
    {
        __attribute__((address_space(3))) uint64_t *lut_lds =
                (__attribute__((address_space(3))) uint64_t *)(uintptr_t)bt_lds_addr(sk_smem);
        for (uint32_t v = threadIdx.x; v < 256u * BT_LUT_COPIES / 8u; v += blockDim.x) {
            const uint32_t b = v & 255u, c0 = 8u * (v >> 8);
            const uint2 e = bt_lut_entry(b);
            const uint64_t e64 = ((uint64_t)e.y << 32) | e.x;
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) lut_lds[b * BT_LUT_COPIES + c0 + ((k + v) & 7u)] = e64;
        }
    }

    bt_v4i acc[SK_NBS_MAX][NB];
#pragma unroll
    for (int i = 0; i < SK_NBS_MAX; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[i][nb] = bt_v4i{0, 0, 0, 0};

    for (int cs = pl.ts; cs < pl.te; cs += CT) {
        const int ce = min(pl.te, cs + CT);
        const int t0 = cs + (wave * 4 + q) * TPL;                // this lane's first tile
        // (1) row segments of the chunk (lane r holds row r's, for every block)
        uint2 seg_e[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i)
            seg_e[i] = sk_segment(ors, i * 16 + r, i < pl.nb_here && i * 16 + r < set_rows, T, cs, ce);
        // (2) this lane's words (tiles past the chunk or the row are cleared)
        uint64_t words[SK_NBS_MAX][TPL];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            const int rr = i * 16 + r;
            const bool ok = i < pl.nb_here && rr < set_rows && t0 < ce;
            const uint32_t off = ok ? ((uint32_t)rr * (uint32_t)T + (uint32_t)t0) * 8u : 0xFFFFFFF0u;
            const uint64_t w0 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off, 0, 0));
            const uint64_t w1 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off + 8u, 0, 0));
            words[i][0] = w0;
            words[i][1] = t0 + 1 < ce ? w1 : 0ull;
        }
        // (3) this lane's X slices for the chunk (zeros past N, past the chunk)
        uint32_t xw[NB][TPL][8];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < TPL; ++k) {
                const int n = r + 16 * nb;
                const uint32_t off = (n < N && t0 + k < ce) ? (uint32_t)n * xs + (uint32_t)(t0 + k) * 32u : 0xFFFFFFE0u;
                const bt_v4i v0 = bt_load_x16<XU>(xrs, off);
                const bt_v4i v1 = bt_load_x16<XU>(xrs, off + 16u);
                xw[nb][k][0] = v0.x; xw[nb][k][1] = v0.y; xw[nb][k][2] = v0.z; xw[nb][k][3] = v0.w;
                xw[nb][k][4] = v1.x; xw[nb][k][5] = v1.y; xw[nb][k][6] = v1.z; xw[nb][k][7] = v1.w;
            }
        // (4) granules of each segment, a block's fit, and the DMAs: segment
        // (i, r) is instruction-slot range [(i 16 + r) iseg, +iseg), its
        // instruction k moves granules 64 k .. 64 k + 63 of the segment
        uint32_t g0[SK_NBS_MAX], ng[SK_NBS_MAX];
        bool fits[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            g0[i] = seg_e[i].x >> 5;
            // the windows of the last tile reach 15 nibbles past the segment's
            // end; an empty segment moves nothing
            ng[i] = seg_e[i].y > seg_e[i].x ? ((seg_e[i].y + 15u) >> 5) - g0[i] + 1u : 0u;
            const uint64_t over = __ballot(r < 16 && ng[i] > (uint32_t)a.iseg * 64u);
            fits[i] = over == 0ull;                                   // wave-uniform (every wavefront loads the same rows)
        }
        const int nins = pl.nb_here * 16 * a.iseg;
        for (int ins = wave; ins < nins; ins += nwaves) {          // wave-uniform loop
            const int seg_i = ins / a.iseg, k = ins - seg_i * a.iseg;
            const int i = seg_i >> 4, rr = seg_i & 15;
            uint32_t sg0 = 0, sng = 0;
            bool fit = false;
#pragma unroll
            for (int ii = 0; ii < SK_NBS_MAX; ++ii)
                if (ii == i) {
                    sg0 = (uint32_t)__builtin_amdgcn_readlane((int)g0[ii], rr);
                    sng = (uint32_t)__builtin_amdgcn_readlane((int)ng[ii], rr);
                    fit = fits[ii];
                }
            const uint32_t u = (uint32_t)k * 64u + (uint32_t)lane;
            uint8_t *dst = slots + (uint32_t)seg_i * slot_bytes + (uint32_t)k * 1024u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)dst, 16,
                                                     (fit && u < sng) ? (sg0 + u) * 16u : 0xFFFFFFF0u, 0, 0, BT_NT);
        }
        // (5) segment popcounts of this lane's tiles, the lane-group prefix,
        // the wavefront's row totals
        uint32_t segc[SK_NBS_MAX], incl[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            segc[i] = (uint32_t)__builtin_popcountll(words[i][0]) + (uint32_t)__builtin_popcountll(words[i][1]);
            uint32_t c = segc[i];
            const uint32_t u16 = (uint32_t)__shfl_up((int)c, 16, 64);
            c += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)c, 32, 64);
            c += q >= 2 ? u32 : 0u;
            incl[i] = c;
            if (q == 3) wt[(i * 16 + r) * nwaves + wave] = (int32_t)c;
        }
        bt_v4i xb[NB][TPL][4];
        bt_make_b<NB, TPL>(xw, xb);
        bt_wait_vm(0);
        __syncthreads();
        // (6) decode + contract every block of the set
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            if (i >= pl.nb_here) break;
            uint32_t before_w = 0;
            for (int w = 0; w < wave; ++w) before_w += (uint32_t)wt[(i * 16 + r) * nwaves + w];
            const uint32_t within = before_w + (incl[i] - segc[i]);   // nibbles of the segment before this lane's tiles
            if (fits[i]) {
                const uint32_t slot = bt_lds_addr(slots) + (uint32_t)(i * 16 + r) * slot_bytes;
                // a corrupt stream stays inside the slot
                const uint32_t local = min((seg_e[i].x & 31u) + within, 2u * (uint32_t)a.iseg * 1024u - 16u - segc[i]);
                bt_contract<NB, TPL>(words[i], local + 2u * slot, BtWinLds{}, lut_base, xb, acc[i]);
            } else {
                bt_contract<NB, TPL>(words[i], seg_e[i].x + within, BtWinGlobal{prs, 0u}, lut_base, xb, acc[i]);
            }
        }
        __syncthreads();   // the slots and row totals are reused by the next chunk
    }

    // the wavefronts' partials (each exact after >> 8) meet in LDS
#pragma unroll
    for (int i = 0; i < SK_NBS_MAX; ++i) {
        if (i >= pl.nb_here) break;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *(__attribute__((address_space(3))) bt_v4i *)(uintptr_t)bt_lds_addr(part + ((i * nwaves + wave) * NB + nb) * 256 + lane * 4) =
                    bt_v4i{acc[i][nb][0] >> 8, acc[i][nb][1] >> 8, acc[i][nb][2] >> 8, acc[i][nb][3] >> 8};
    }
    __syncthreads();
    // item (block i, column n, row group): 4 consecutive rows of column n;
    // D layout of the 16x16 MFMAs: lane l, register k -> row 4 (l / 16) + k, column l % 16
    int32_t *wsp = reinterpret_cast<int32_t *>(a.ws_part);
    const int items = pl.nb_here * NB * 64;
    for (int o = threadIdx.x; o < items; o += blockDim.x) {
        const int i = o / (NB * 64), nb = (o / 64) % NB, ln = o % 64;
        const int n = (ln & 15) + 16 * nb;
        if (n >= N) continue;
        bt_v4i s = bt_v4i{0, 0, 0, 0};
        for (int w = 0; w < nwaves; ++w)
            s += *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(part + ((i * nwaves + w) * NB + nb) * 256 + ln * 4);
        const int b = pl.b0 + i;
        const int rl = 4 * (ln >> 4);
        if (a.S == 1) {
            const int m = b * 16 + rl;
            int32_t *y = reinterpret_cast<int32_t *>(a.Y) + (int64_t)n * M + m;
            const int32_t v[4] = {s.x, s.y, s.z, s.w};
            for (int k = 0; k < 4 && m + k < M; ++k) y[k] = v[k];
        } else {
            int32_t *w = wsp + (((int64_t)b * a.S + pl.split) * N + n) * 16 + rl;
            sk_ws_store(w, s.x);
            sk_ws_store(w + 1, s.y);
            sk_ws_store(w + 2, s.z);
            sk_ws_store(w + 3, s.w);
        }
    }
    if (a.S == 1) return;
    if (!sk_last_arrival(a, pl, flag)) return;
    for (int o = threadIdx.x; o < pl.nb_here * 16 * N; o += blockDim.x) {
        const int i = o / (16 * N), n = (o / 16) % N, rl = o % 16;
        const int b = pl.b0 + i, m = b * 16 + rl;
        if (m >= M) continue;
        int32_t s = 0;
        for (int sp = 0; sp < a.S; ++sp) s += sk_ws_load(wsp + (((int64_t)b * a.S + sp) * N + n) * 16 + rl);
        reinterpret_cast<int32_t *>(a.Y)[(int64_t)n * M + m] = s;
    }
    sk_reset(a, pl);   // ready for the next call
}

// LDS of the int4 kernel; the partials ([nbs][nwaves][nb][256] ints) reuse
// the slots, which are never smaller (16 (1 KB + 64) >= 8 x 2 x 1 KB)
static size_t bsk_w4a4_lds(int nwaves, int nbs, int iseg) {
    return (size_t)BT_LUT_BYTES + (size_t)SK_NBS_MAX * 16 * nwaves * 4 +
           (size_t)nbs * 16 * ((size_t)iseg * 1024 + SK_SLOT_SKEW) + 16;
}

// ------------------------------------------------------------ int4, streamed

// The same work item walked as the streaming kernel walks its blocks: a set
// of at most SKS_NBLK blocks over one K range of at most 32 TPL tiles (eight
// wavefronts, TPL tiles per lane), the block's range of every row decoded in
// one pass, and block i + 1's row segments in flight while block i is
// decoded. Per block:
//   - its 16 row segments (their ends read from the format's offsets for
//     every block of the set at the start, with X and block 0's words) go
//     by DMA to slots of their own, ISEG KB each plus 48 bytes (every row
//     starts 12 banks further round than the one before it), 2 ISEG
//     instructions per wavefront; a block with a segment longer than its
//     slot reads its windows from global memory instead (every wavefront
//     decides alike);
//   - once it has landed and every wavefront has posted its row totals (one
//     barrier), a lane's start is its segment's first nibble inside the
//     first granule plus the tiles before its own in the row's range;
//   - the next block's words and segments are issued before that barrier, so
//     one transfer is in flight while each block is decoded.
// Partials and the reduction are those of k_bsk_w4a4.
#define SKS_NBLK 3
#define SKS_SKEW 48u
#define SKS_WAVES 8

// LDS of the streamed kernel: selector table | row totals [NBLK][16][8] |
// partials [nbs][8][NB * 256] ints | slots [nbs][16][ISEG KB + 48] | flag
static size_t bsks_w4a4_lds(int nb, int nbs, int iseg) {
    return (size_t)BT_LUT_BYTES + (size_t)SKS_NBLK * 16 * SKS_WAVES * 4 + (size_t)nbs * SKS_WAVES * nb * 1024 +
           (size_t)nbs * 16 * ((size_t)iseg * 1024 + SKS_SKEW) + 16;
}

template <int NB, int TPL, int ISEG, bool XU>
__global__ __launch_bounds__(512) void k_bsks_w4a4(SkArgs a) {
    constexpr int WC = SKS_WAVES, D = 16 * ISEG / SKS_WAVES;   // DMA instructions per wavefront and block
    extern __shared__ __attribute__((aligned(16))) uint8_t sk_smem[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int M = a.M, T = a.T, N = a.N;
    const SkPlace pl = sk_place(a);
    const int nblk = pl.nb_here;                       // 1 .. SKS_NBLK
    const int tr = pl.te - pl.ts;                      // tiles of the range, <= 32 TPL
    const int t0 = (wave * 4 + q) * TPL;               // this lane's first tile, from the range's start
    const uint32_t xs = ((uint32_t)a.K + 1u) >> 1;
    constexpr uint32_t slot_bytes = (uint32_t)ISEG * 1024u + SKS_SKEW;
    constexpr uint32_t cap = (uint32_t)ISEG * 64u;     // granules a slot holds

    const uint32_t lut_base = bt_lds_addr(sk_smem) + (uint32_t)(lane % BT_LUT_COPIES) * 8u;
    int32_t *wt = reinterpret_cast<int32_t *>(sk_smem + BT_LUT_BYTES);
    int32_t *part = wt + SKS_NBLK * 16 * WC;
    uint8_t *slots = reinterpret_cast<uint8_t *>(part + a.nbs * WC * NB * 256);
    int *flag = reinterpret_cast<int *>(slots + (uint32_t)a.nbs * 16u * slot_bytes);

    const int set_rows = min(nblk * 16, M - pl.b0 * 16);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(a.payload, a.payload_bytes);
    const __amdgpu_buffer_rsrc_t ors = bt_rsrc(a.offsets + (int64_t)pl.b0 * 16 * T, ((uint32_t)set_rows * (uint32_t)T + 1u) * 4u);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(a.bitmaps + (int64_t)pl.b0 * 16 * T, (uint32_t)set_rows * (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(a.X, bt_x_range(N, xs));
    asm volatile("" ::"s"(a.payload), "s"(a.X), "s"(a.Y), "s"(N));

    // (1) every block's row segments (lane r: row r of each block), first
    uint2 seg[SKS_NBLK];
#pragma unroll
    for (int i = 0; i < SKS_NBLK; ++i)
        seg[i] = sk_segment(ors, i * 16 + r, i < nblk && i * 16 + r < set_rows, T, pl.ts, pl.te);
    // (2) X slices of the lane's tiles (zeros past N or past the range)
    uint32_t xw[NB][TPL][8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int k = 0; k < TPL; ++k) {
            const int n = r + 16 * nb;
            const uint32_t off =
                    (n < N && t0 + k < tr) ? (uint32_t)n * xs + (uint32_t)(pl.ts + t0 + k) * 32u : 0xFFFFFFE0u;
            const bt_v4i v0 = bt_load_x16<XU>(xrs, off);
            const bt_v4i v1 = bt_load_x16<XU>(xrs, off + 16u);
            xw[nb][k][0] = v0.x; xw[nb][k][1] = v0.y; xw[nb][k][2] = v0.z; xw[nb][k][3] = v0.w;
            xw[nb][k][4] = v1.x; xw[nb][k][5] = v1.y; xw[nb][k][6] = v1.z; xw[nb][k][7] = v1.w;
        }
    // (3) words: block 0's now, block i + 1's with its segments (tiles past
    // the range are cleared before use; rows past the set read zeros)
    uint64_t words[SKS_NBLK][TPL];
    auto load_words = [&](int i) -> void {
        const int rr = i * 16 + r;
        const uint32_t off = ((uint32_t)rr * (uint32_t)T + (uint32_t)(pl.ts + t0)) * 8u;
        const bt_v4i v = __builtin_bit_cast(bt_v4i, __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, BT_NT));
        words[i][0] = ((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x;
        words[i][1] = ((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z;
        if constexpr (TPL == 3)
            words[i][2] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off + 16u, 0, BT_NT));
    };
    load_words(0);
    // (4) each block's granules and whether its segments fit their slots
    uint32_t g0[SKS_NBLK], ng[SKS_NBLK];
    bool fits[SKS_NBLK];
#pragma unroll
    for (int i = 0; i < SKS_NBLK; ++i) {
        g0[i] = seg[i].x >> 5;
        // the windows of a row's last tile reach 15 nibbles past its segment
        ng[i] = seg[i].y > seg[i].x ? ((seg[i].y + 15u) >> 5) - g0[i] + 1u : 0u;
        fits[i] = __ballot(ng[i] > cap) == 0ull;   // wave-uniform: every wavefront holds the same rows
    }
    // block i's DMAs: instruction j = wave + 8 d moves KB j % ISEG of row
    // j / ISEG's segment (a fixed count per wavefront, so the compiler's own
    // waits stay exact)
    auto issue = [&](int i) -> void {
        uint8_t *buf = slots + (uint32_t)i * 16u * slot_bytes;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int j = wave + SKS_WAVES * d;
            const int row = j / ISEG, k = j - row * ISEG;
            uint32_t sg0 = 0, sng = 0;
#pragma unroll
            for (int ii = 0; ii < SKS_NBLK; ++ii)
                if (ii == i) {
                    sg0 = (uint32_t)__builtin_amdgcn_readlane((int)g0[ii], row);
                    sng = fits[ii] ? (uint32_t)__builtin_amdgcn_readlane((int)ng[ii], row) : 0u;
                }
            const uint32_t u = (uint32_t)k * 64u + (uint32_t)lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)(buf + (uint32_t)row * slot_bytes + (uint32_t)k * 1024u),
                                                     16, u < sng ? (sg0 + u) * 16u : 0xFFFFFFF0u, 0, 0, BT_NT);
        }
    };
    issue(0);
    {
        __attribute__((address_space(3))) uint64_t *lut_lds =
                (__attribute__((address_space(3))) uint64_t *)(uintptr_t)bt_lds_addr(sk_smem);
        for (uint32_t v = threadIdx.x; v < 256u * BT_LUT_COPIES / 8u; v += blockDim.x) {
            const uint32_t b = v & 255u, c0 = 8u * (v >> 8);
            const uint2 e = bt_lut_entry(b);
            const uint64_t e64 = ((uint64_t)e.y << 32) | e.x;
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) lut_lds[b * BT_LUT_COPIES + c0 + ((k + v) & 7u)] = e64;
        }
    }

    bt_v4i xb[NB][TPL][4];
#pragma unroll
    for (int i = 0; i < SKS_NBLK; ++i) {
        if (i >= nblk) break;
#pragma unroll
        for (int k = 0; k < TPL; ++k)
            if (t0 + k >= tr) words[i][k] = 0;
        uint32_t sc = 0;
#pragma unroll
        for (int k = 0; k < TPL; ++k) sc += (uint32_t)__builtin_popcountll(words[i][k]);
        uint32_t incl = sc;
        {
            const uint32_t u16 = (uint32_t)__shfl_up((int)incl, 16, 64);
            incl += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)incl, 32, 64);
            incl += q >= 2 ? u32 : 0u;
        }
        int32_t *wti = wt + i * 16 * WC;
        if (q == 3) wti[r * WC + wave] = (int32_t)incl;
        bt_wait_vm(0);   // this wavefront's share of block i landed (nothing later is in flight)
        if (i + 1 < nblk) {
            load_words(i + 1);
            issue(i + 1);
        }
        if (i == 0) bt_make_b<NB, TPL>(xw, xb);
        bt_barrier_lds();   // ... everyone's, and every row total of block i
        uint32_t before_w;
        {
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
            before_w = pre[wave];
        }
        const uint32_t within = before_w + (incl - sc);   // nibbles of the row's range before this lane's tiles
        bt_v4i acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = bt_v4i{0, 0, 0, 0};
        if (fits[i]) {
            const uint32_t slot = bt_lds_addr(slots + (uint32_t)(i * 16 + r) * slot_bytes);
            // a corrupt stream stays inside the slot
            const uint32_t local = min((seg[i].x & 31u) + within, 2u * (uint32_t)ISEG * 1024u - 16u - sc);
            bt_contract<NB, TPL>(words[i], local + 2u * slot, BtWinLds{}, lut_base, xb, acc);
        } else {
            bt_contract<NB, TPL>(words[i], seg[i].x + within, BtWinGlobal{prs, 0u}, lut_base, xb, acc);
        }
        int32_t *pw = part + (i * WC + wave) * NB * 256;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            *(__attribute__((address_space(3))) bt_v4i *)(uintptr_t)bt_lds_addr(pw + nb * 256 + lane * 4) =
                    bt_v4i{acc[nb][0] >> 8, acc[nb][1] >> 8, acc[nb][2] >> 8, acc[nb][3] >> 8};
    }
    bt_barrier_lds();
    // item (block i, column block nb, lane l): rows 4 (l / 16) .. +3 of
    // column l % 16 (the MFMA D layout), the wavefronts' partials added in order
    int32_t *wsp = reinterpret_cast<int32_t *>(a.ws_part);
    for (int o = threadIdx.x; o < nblk * NB * 64; o += blockDim.x) {
        const int i = o / (NB * 64), nb = (o / 64) % NB, ln = o % 64;
        const int n = (ln & 15) + 16 * nb;
        if (n >= N) continue;
        bt_v4i sum = bt_v4i{0, 0, 0, 0};
        for (int w = 0; w < WC; ++w)
            sum += *(bt_lds_v4i *)(uintptr_t)bt_lds_addr(part + ((i * WC + w) * NB + nb) * 256 + ln * 4);
        const int b = pl.b0 + i, rl = 4 * (ln >> 4);
        if (a.S == 1) {
            const int m = b * 16 + rl;
            int32_t *y = reinterpret_cast<int32_t *>(a.Y) + (int64_t)n * M + m;
            const int32_t v[4] = {sum.x, sum.y, sum.z, sum.w};
            for (int k = 0; k < 4 && m + k < M; ++k) y[k] = v[k];
        } else {
            int32_t *w = wsp + (((int64_t)b * a.S + pl.split) * N + n) * 16 + rl;
            sk_ws_store(w, sum.x);
            sk_ws_store(w + 1, sum.y);
            sk_ws_store(w + 2, sum.z);
            sk_ws_store(w + 3, sum.w);
        }
    }
    if (a.S == 1) return;
    if (!sk_last_arrival(a, pl, flag)) return;
    for (int o = threadIdx.x; o < nblk * 16 * N; o += blockDim.x) {
        const int i = o / (16 * N), n = (o / 16) % N, rl = o % 16;
        const int b = pl.b0 + i, m = b * 16 + rl;
        if (m >= M) continue;
        int32_t v = 0;
        for (int sp = 0; sp < a.S; ++sp) v += sk_ws_load(wsp + (((int64_t)b * a.S + sp) * N + n) * 16 + rl);
        reinterpret_cast<int32_t *>(a.Y)[(int64_t)n * M + m] = v;
    }
    sk_reset(a, pl);
}

// ------------------------------------------------------------------ fp16

// Same skeleton with one tile per lane (CT = 4 x wavefronts), u16 payload
// (8 elements per 16-byte granule), the fp16 decode and MFMA of the 16-row
// kernel, fp32 partials, and one round-to-nearest-even to fp16 at the end.
template <int NB>
__global__ __launch_bounds__(1024) void k_bsk_f16(SkArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t sk_smem[];
    const int nwaves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, q = lane >> 4;
    const int M = a.M, K = a.K, T = a.T, N = a.N;
    const int CT = 4 * nwaves;                                   // tiles per chunk
    const SkPlace pl = sk_place(a);
    const uint32_t slot_bytes = (uint32_t)a.iseg * 1024u + SK_SLOT_SKEW;

    // LDS: selector table (16 entries) | row totals [NBS_MAX][16][nwaves] |
    // segment slots [nbs][16] (after the last chunk: the wavefronts' fp32
    // partials [nbs][nwaves][NB * 256]) | flag
    uint32_t *lut_lds = reinterpret_cast<uint32_t *>(sk_smem);
    int32_t *wt = reinterpret_cast<int32_t *>(sk_smem + 128);
    uint8_t *slots = reinterpret_cast<uint8_t *>(wt + SK_NBS_MAX * 16 * nwaves);
    float *part = reinterpret_cast<float *>(slots);
    const uint32_t slot_region = max((uint32_t)a.nbs * 16u * slot_bytes, (uint32_t)(a.nbs * nwaves * NB) * 1024u);
    int *flag = reinterpret_cast<int *>(slots + slot_region);
    const uint32_t lut = bt_lds_addr(lut_lds);

    const int set_rows = min(pl.nb_here * 16, M - pl.b0 * 16);
    const __amdgpu_buffer_rsrc_t prs = bt_rsrc(a.payload, a.payload_bytes);
    const __amdgpu_buffer_rsrc_t ors = bt_rsrc(a.offsets + (int64_t)pl.b0 * 16 * T, ((uint32_t)set_rows * (uint32_t)T + 1u) * 4u);
    const __amdgpu_buffer_rsrc_t brs = bt_rsrc(a.bitmaps + (int64_t)pl.b0 * 16 * T, (uint32_t)set_rows * (uint32_t)T * 8u);
    const __amdgpu_buffer_rsrc_t xrs = bt_rsrc(a.X, (uint32_t)N * (uint32_t)K * 2u);

    // the 16-entry selector table (entry m: the perm selectors of nibble m)
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

    bf_f4 acc[SK_NBS_MAX][NB];
#pragma unroll
    for (int i = 0; i < SK_NBS_MAX; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[i][nb] = bf_f4{0.f, 0.f, 0.f, 0.f};

    for (int cs = pl.ts; cs < pl.te; cs += CT) {
        const int ce = min(pl.te, cs + CT);
        const int t = cs + wave * 4 + q;                         // this lane's tile
        uint2 seg_e[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i)
            seg_e[i] = sk_segment(ors, i * 16 + r, i < pl.nb_here && i * 16 + r < set_rows, T, cs, ce);
        uint64_t words[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            const int rr = i * 16 + r;
            const bool ok = i < pl.nb_here && rr < set_rows && t < ce;
            const uint32_t off = ok ? ((uint32_t)rr * (uint32_t)T + (uint32_t)t) * 8u : 0xFFFFFFF0u;
            words[i] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(brs, off, 0, 0));
        }
        // this lane's X: column r + 16 nb, positions 64 t .. 64 t + 63 (zeros
        // past N, past the chunk, and past K: a zero weight times a
        // non-finite X from the next row would give NaN)
        bf_h8 xb[NB][8];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = r + 16 * nb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t k0 = (uint32_t)t * 64u + 8u * (uint32_t)j;
                const uint32_t off = (n < N && t < ce && k0 < (uint32_t)K) ? ((uint32_t)n * (uint32_t)K + k0) * 2u
                                                                           : 0xFFFFFFF0u;
                xb[nb][j] = __builtin_bit_cast(bf_h8, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
            }
        }
        uint32_t g0[SK_NBS_MAX], ng[SK_NBS_MAX];
        bool fits[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            g0[i] = seg_e[i].x >> 3;
            // the windows of the last tile reach 5 elements past the segment's end
            ng[i] = seg_e[i].y > seg_e[i].x ? ((seg_e[i].y + 5u) >> 3) - g0[i] + 1u : 0u;
            fits[i] = __ballot(ng[i] > (uint32_t)a.iseg * 64u) == 0ull;
        }
        const int nins = pl.nb_here * 16 * a.iseg;
        for (int ins = wave; ins < nins; ins += nwaves) {
            const int seg_i = ins / a.iseg, k = ins - seg_i * a.iseg;
            const int i = seg_i >> 4, rr = seg_i & 15;
            uint32_t sg0 = 0, sng = 0;
            bool fit = false;
#pragma unroll
            for (int ii = 0; ii < SK_NBS_MAX; ++ii)
                if (ii == i) {
                    sg0 = (uint32_t)__builtin_amdgcn_readlane((int)g0[ii], rr);
                    sng = (uint32_t)__builtin_amdgcn_readlane((int)ng[ii], rr);
                    fit = fits[ii];
                }
            const uint32_t u = (uint32_t)k * 64u + (uint32_t)lane;
            uint8_t *dst = slots + (uint32_t)seg_i * slot_bytes + (uint32_t)k * 1024u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (bt_lds_void *)dst, 16,
                                                     (fit && u < sng) ? (sg0 + u) * 16u : 0xFFFFFFF0u, 0, 0, BT_NT);
        }
        uint32_t segc[SK_NBS_MAX], incl[SK_NBS_MAX];
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            segc[i] = (uint32_t)__builtin_popcountll(words[i]);
            uint32_t c = segc[i];
            const uint32_t u16 = (uint32_t)__shfl_up((int)c, 16, 64);
            c += q >= 1 ? u16 : 0u;
            const uint32_t u32 = (uint32_t)__shfl_up((int)c, 32, 64);
            c += q >= 2 ? u32 : 0u;
            incl[i] = c;
            if (q == 3) wt[(i * 16 + r) * nwaves + wave] = (int32_t)c;
        }
        bt_wait_vm(0);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SK_NBS_MAX; ++i) {
            if (i >= pl.nb_here) break;
            uint32_t before_w = 0;
            for (int w = 0; w < wave; ++w) before_w += (uint32_t)wt[(i * 16 + r) * nwaves + w];
            const uint32_t within = before_w + (incl[i] - segc[i]);   // elements of the segment before this lane's tile
            if (fits[i]) {
                const uint32_t slot = bt_lds_addr(slots) + (uint32_t)(i * 16 + r) * slot_bytes;
                // a corrupt stream stays inside the slot
                const uint32_t local = min((seg_e[i].x & 7u) + within, 512u * (uint32_t)a.iseg - 8u - segc[i]);
                bf_contract<NB>(words[i], local + (slot >> 1), BfWinLds{}, lut, xb, acc[i]);
            } else {
                bf_contract<NB>(words[i], seg_e[i].x + within, BfWinGlobal{prs, 0u}, lut, xb, acc[i]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < SK_NBS_MAX; ++i) {
        if (i >= pl.nb_here) break;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int k = 0; k < 4; ++k) part[((i * nwaves + wave) * NB + nb) * 256 + k * 64 + lane] = acc[i][nb][k];
    }
    __syncthreads();
    // item (block i, column n, row rl): the wavefronts' partials in
    // wavefront order (D layout: lane l, register k -> row 4 (l / 16) + k, column l % 16)
    float *wsp = reinterpret_cast<float *>(a.ws_part);
    uint16_t *Y = reinterpret_cast<uint16_t *>(a.Y);
    for (int o = threadIdx.x; o < pl.nb_here * 16 * N; o += blockDim.x) {
        const int i = o / (16 * N), n = (o / 16) % N, rl = o % 16;
        const int nb = n >> 4, col = n & 15, ln = (rl >> 2) * 16 + col, k = rl & 3;
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += part[((i * nwaves + w) * NB + nb) * 256 + k * 64 + ln];
        const int b = pl.b0 + i, m = b * 16 + rl;
        if (a.S == 1) {
            if (m < M) Y[(int64_t)n * M + m] = __builtin_bit_cast(uint16_t, (_Float16)s);
        } else {
            sk_ws_store(wsp + (((int64_t)b * a.S + pl.split) * N + n) * 16 + rl, s);
        }
    }
    if (a.S == 1) return;
    if (!sk_last_arrival(a, pl, flag)) return;
    for (int o = threadIdx.x; o < pl.nb_here * 16 * N; o += blockDim.x) {
        const int i = o / (16 * N), n = (o / 16) % N, rl = o % 16;
        const int b = pl.b0 + i, m = b * 16 + rl;
        if (m >= M) continue;
        float s = 0.f;
        for (int sp = 0; sp < a.S; ++sp) s += sk_ws_load(wsp + (((int64_t)b * a.S + sp) * N + n) * 16 + rl);
        Y[(int64_t)n * M + m] = __builtin_bit_cast(uint16_t, (_Float16)s);
    }
    sk_reset(a, pl);
}

// LDS of the fp16 kernel; the fp32 partials ([nbs][nwaves][nb][256]) reuse
// the slots (16 (1 KB iseg + 64) >= 16 x 2 x 1 KB needs iseg >= 2 at 16
// wavefronts and N > 16: the plan takes the larger of the two)
static size_t bsk_f16_lds(int nwaves, int nb, int nbs, int iseg) {
    const size_t slots = (size_t)nbs * 16 * ((size_t)iseg * 1024 + SK_SLOT_SKEW);
    const size_t parts = (size_t)nbs * nwaves * nb * 256 * 4;
    return 128 + (size_t)SK_NBS_MAX * 16 * nwaves * 4 + (slots > parts ? slots : parts) + 16;
}

// ------------------------------------------------------------------ host

struct SkPlan {
    int dtype;          // BSP_INT4 or BSP_FP16
    int nwaves, nb;     // wavefronts per workgroup; column blocks of 16 (N <= 16: 1)
    int nbs, S, tps;    // blocks per set, splits per set, tiles per split
    int iseg;           // KB of LDS slot per row segment
    int nsets;
    unsigned grid;
    size_t lds;
    int64_t ws_bytes;   // workspace the plan needs (0 for S == 1)
    int streamed = 0;   // k_bsks_w4a4 (int4, one pass per block and range) instead of k_bsk_*
    int tpl = 2;        // streamed: tiles per lane
};

// Workspace layout: a fixed area of arrival counters (one uint32 per set,
// zero between calls) first, then the partial sums. The counter area's size
// does not depend on the problem, so the partials of one call never land on
// counters another call of a different shape uses on the same workspace.
#define SK_WS_COUNTERS 16384
static int64_t sk_ws_counters_bytes() { return (int64_t)SK_WS_COUNTERS * 4; }

// Plan for the K-range kernels. splits: 1 (no workspace: one workgroup walks
// all of K of a block in chunks) or the number of K ranges per block set (2
// or 4; then the set holds as many blocks, so that a workgroup decodes one
// block's worth of weights with 1 / splits of X). Returns false if the shape
// is outside (N > 32, K >= 2^25, or an LDS plan that does not fit).
static bool sk_plan(int dtype, int64_t M, int64_t K, int64_t N, int64_t payload_bytes, int splits, SkPlan *p) {
    if (M <= 0 || K <= 0 || N < 1 || N > 32 || splits < 1 || splits > SK_NBS_MAX) return false;
    const int64_t T = (K + 63) / 64, blocks = (M + 15) / 16;
    if (splits > 1 && T < 2 * splits) return false;               // at least two tiles per split
    if (M * T + 1 > (int64_t)UINT32_MAX / 8) return false;        // 32-bit buffer ranges of words and offsets
    p->dtype = dtype;
    p->nb = N <= 16 ? 1 : 2;
    p->S = splits;
    // blocks per set: as many as K ranges, or one for fp16 at N <= 8 (more,
    // smaller workgroups that share the CUs; 4096 x 11008 at N = 1 with 2
    // ranges 25.6 -> 22.1 us, N = 8 27.7 -> 24.7, 4096 x 13824 33.0 -> 27.6,
    // 11008 x 11008 72.1 -> 57.7) while one counter per block is left; at
    // larger N each workgroup's reads of X outweigh that (N = 16 32.6 ->
    // 36.0, N = 32 50.6 -> 64.5)
    p->nbs = dtype == BSP_FP16 && N <= 8 && blocks <= SK_WS_COUNTERS ? 1 : splits;
    if (splits > 1 && (blocks + p->nbs - 1) / p->nbs > SK_WS_COUNTERS) return false;   // one counter per set
    p->nsets = (int)((blocks + p->nbs - 1) / p->nbs);
    p->tps = (int)((T + splits - 1) / splits);
    const int per_wave = dtype == BSP_INT4 ? 8 : 4;                 // tiles per wavefront and chunk
    const int max_waves = dtype == BSP_INT4 ? 8 : 16;
    // wavefronts: enough for the split's tiles, fewer (shorter chunks, smaller
    // slots) when the slots of a dense set would not fit the LDS
    int nw = (int)std::min<int64_t>(max_waves, (std::min<int64_t>(p->tps, (int64_t)per_wave * max_waves) + per_wave - 1) / per_wave);
    // fp16 past 256 workgroups: shorter chunks (at least 4 wavefronts) so
    // that up to 4 workgroups share a CU instead of running in rounds of one
    // (N = 1: 5120 x 5120 34.2 -> 20.2 us, 13824 x 5120 66.7 -> 33.2, 5120 x
    // 13824 65.9 -> 40.8, 8192 x 8192 36.9 -> 27.1; N = 8 42.1 -> 30.8); a
    // second pass takes the whole LDS when that fails
    const int64_t wg_per_cu =
            dtype == BSP_FP16 ? std::min<int64_t>(4, ((int64_t)p->nsets * p->S + BT_CUS - 1) / BT_CUS) : 1;
    for (int pass = 0;; nw = nw > 1 ? nw / 2 : 0) {
        if (nw == 0) {
            if (pass == 1 || wg_per_cu == 1) return false;
            pass = 1;
            nw = (int)std::min<int64_t>(max_waves, (std::min<int64_t>(p->tps, (int64_t)per_wave * max_waves) + per_wave - 1) / per_wave);
        }
        const int64_t ct = (int64_t)per_wave * nw;
        // slot per row segment: the average segment of a chunk, +30 % and
        // 64 B of windows and granule alignment (at most a dense segment); a
        // block with a longer one reads its windows from global memory
        const int64_t seg_avg = payload_bytes * std::min<int64_t>(ct, T) / std::max<int64_t>(M * T, 1);
        const int64_t seg_max = dtype == BSP_INT4 ? ct * 32 : ct * 128;
        const int iseg = (int)std::max<int64_t>(1, (std::min(seg_avg + seg_avg * 3 / 10, seg_max) + 64 + 1023) / 1024);
        const size_t lds = dtype == BSP_INT4 ? bsk_w4a4_lds(nw, p->nbs, iseg) : bsk_f16_lds(nw, p->nb, p->nbs, iseg);
        if (lds <= (size_t)(160 * 1024 / (pass ? 1 : wg_per_cu)) && (pass || nw >= 4 || wg_per_cu == 1)) {
            p->nwaves = nw;
            p->iseg = iseg;
            p->lds = lds;
            break;
        }
    }
    p->grid = (unsigned)(p->nsets * p->S);
    const int64_t esize = 4;                                          // int32 or fp32 partials
    p->ws_bytes = splits > 1 ? sk_ws_counters_bytes() + (int64_t)p->nsets * p->nbs * p->S * N * 16 * esize : 0;
    return true;
}

// Plan for the streamed int4 kernel: S >= 2 K ranges of at most 32 TPL
// tiles (TPL 2 or 3), sets of at most SKS_NBLK blocks, and no more
// workgroups than CUs (each holds most of the LDS, so a workgroup past the
// CU count would wait for a whole one to finish): the fewest blocks per set
// that allow it. Slots of one KB per row segment when the average segment
// plus 30 % and 64 B of windows fits one, else two; a block with a longer
// segment reads its windows from global memory.
static bool sks_plan(int64_t M, int64_t K, int64_t N, int64_t payload_bytes, int S, SkPlan *p) {
    if (M <= 0 || K <= 0 || N < 1 || N > 32 || S < 2 || S > SK_NBS_MAX) return false;
    const int64_t T = (K + 63) / 64, blocks = (M + 15) / 16;
    if (M * T + 1 > (int64_t)UINT32_MAX / 8) return false;          // 32-bit buffer ranges of words and offsets
    {
        const int64_t tps = (T + S - 1) / S;
        if (tps < 2 || (S - 1) * tps >= T) return false;              // every split holds tiles
        const int tpl = tps <= 64 ? 2 : 3;
        if (tps > 32 * tpl) return false;
        for (int nbs = 1; nbs <= SKS_NBLK; ++nbs) {
            const int64_t nsets = (blocks + nbs - 1) / nbs;
            if (nsets * S > BT_CUS || nsets > SK_WS_COUNTERS) continue;
            const int64_t seg_avg = payload_bytes * tps / std::max<int64_t>(M * T, 1);
            const int iseg = seg_avg + seg_avg * 3 / 10 + 64 <= 1024 ? 1 : 2;
            const int nb = N <= 16 ? 1 : 2;
            const size_t lds = bsks_w4a4_lds(nb, nbs, iseg);
            if (lds > 160 * 1024) continue;
            p->dtype = BSP_INT4;
            p->nwaves = SKS_WAVES;
            p->nb = nb;
            p->nbs = nbs;
            p->S = S;
            p->tps = (int)tps;
            p->iseg = iseg;
            p->nsets = (int)nsets;
            p->grid = (unsigned)(nsets * S);
            p->lds = lds;
            p->ws_bytes = sk_ws_counters_bytes() + nsets * nbs * S * N * 16 * 4;
            p->streamed = 1;
            p->tpl = tpl;
            return true;
        }
    }
    return false;
}

static SkArgs sk_args(const SkPlan &p, const uint64_t *bitmaps, const uint32_t *offsets, const void *payload,
                      uint32_t payload_bytes, int M, int K, const void *X, int N, void *Y, void *workspace) {
    SkArgs a;
    a.bitmaps = bitmaps; a.offsets = offsets; a.payload = payload; a.payload_bytes = payload_bytes;
    a.M = M; a.K = K; a.N = N; a.T = (K + 63) / 64; a.X = X; a.Y = Y;
    a.nbs = p.nbs; a.nsets = p.nsets; a.S = p.S; a.tps = p.tps; a.iseg = p.iseg;
    a.ws_cnt = reinterpret_cast<uint32_t *>(workspace);
    a.ws_part = workspace ? reinterpret_cast<uint8_t *>(workspace) + sk_ws_counters_bytes() : nullptr;
    return a;
}

template <int NB, int TPL, int ISEG, bool XU>
static void launch_bsks_t(const SkPlan &p, const SkArgs &a, hipStream_t stream) {
    (void)hipFuncSetAttribute((const void *)k_bsks_w4a4<NB, TPL, ISEG, XU>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)p.lds);
    hipLaunchKernelGGL((k_bsks_w4a4<NB, TPL, ISEG, XU>), dim3(p.grid), dim3(64 * SKS_WAVES), p.lds, stream, a);
}

template <int NB, int TPL>
static void launch_bsks_i(const SkPlan &p, const SkArgs &a, bool xu, hipStream_t stream) {
    if (p.iseg == 1) { if (xu) launch_bsks_t<NB, TPL, 1, true>(p, a, stream); else launch_bsks_t<NB, TPL, 1, false>(p, a, stream); }
    else { if (xu) launch_bsks_t<NB, TPL, 2, true>(p, a, stream); else launch_bsks_t<NB, TPL, 2, false>(p, a, stream); }
}

static void launch_bsk(const SkPlan &p, const SkArgs &a, hipStream_t stream) {
    const dim3 grid(p.grid), block(64 * p.nwaves);
    if (p.streamed) {
        const bool xu = a.K % 8 != 0;
        if (p.nb == 1) { if (p.tpl == 2) launch_bsks_i<1, 2>(p, a, xu, stream); else launch_bsks_i<1, 3>(p, a, xu, stream); }
        else { if (p.tpl == 2) launch_bsks_i<2, 2>(p, a, xu, stream); else launch_bsks_i<2, 3>(p, a, xu, stream); }
        return;
    }
    if (p.dtype == BSP_INT4) {
        const bool xu = a.K % 8 != 0;
#define SK_L4(NB, XU)                                                                                       \
    do {                                                                                                    \
        (void)hipFuncSetAttribute((const void *)k_bsk_w4a4<NB, XU>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                  (int)p.lds);                                                              \
        hipLaunchKernelGGL((k_bsk_w4a4<NB, XU>), grid, block, p.lds, stream, a);                           \
    } while (0)
        if (p.nb == 1) { if (xu) SK_L4(1, true); else SK_L4(1, false); }
        else { if (xu) SK_L4(2, true); else SK_L4(2, false); }
#undef SK_L4
    } else {
        if (p.nb == 1) {
            (void)hipFuncSetAttribute((const void *)k_bsk_f16<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
            hipLaunchKernelGGL((k_bsk_f16<1>), grid, block, p.lds, stream, a);
        } else {
            (void)hipFuncSetAttribute((const void *)k_bsk_f16<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
            hipLaunchKernelGGL((k_bsk_f16<2>), grid, block, p.lds, stream, a);
        }
    }
}
