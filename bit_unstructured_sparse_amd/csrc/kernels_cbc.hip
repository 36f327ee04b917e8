// kernels_cbc.hip -- fp16 decode-phase product with dynamic activation
// pruning over the Tiled-CBC format on gfx950: SPDP, Sec. 4.1 (Tiled-CBC)
// and Sec. 4.2 (the spMspV kernel and its HAD-SMBD decoding).
//
// Y[n][m] = sum over k of W[m][k] * x'[n][k], x' = x where |x| > tau, else 0.
// A column k whose activations are all pruned is skipped: its bitmap words
// and values are never read, which is where dynamic pruning saves bytes.
//
// Work split. Rows go in bands of 256 (one column tile of a GTile); a
// workgroup of 4 wavefronts takes one band and a segment of G consecutive
// GTiles (G x 64 columns); wavefront w owns rows 64 w .. 64 w + 63 of the
// band, one per lane (the column-major, CUDA-core style register layout of
// HAD-SMBD: one output row per thread, one column at a time).
//
// A workgroup first stages its segment of X, applies the threshold and
// builds the list of active columns in LDS (ballot and prefix count). Then,
// for each active column, every wavefront reads the column's four bitmap
// words, its ColInfo and its GTile's offset with scalar loads (one address
// for the whole wavefront), finds its lane's rank with a masked popcount
// (v_mbcnt over its own word plus the set bits of the words of the lower
// wavefronts) and gathers its value (lanes whose bit is clear read zero
// through the buffer range check), and accumulates value x x' in fp32.
// Eight columns are unrolled so that their loads are in flight together.
//
// Segments of one band meet through a workspace: each workgroup posts its
// fp32 partials, and the last of the band's workgroups to arrive (an
// agent-scope counter) adds the segments in segment order (so the result
// does not depend on timing) and writes Y in fp16 (round to nearest even).
// Without a workspace one workgroup covers the whole band, CBC_SEG_MAX
// GTiles at a time.

#define CBC_TM BSP_CBC_TILE_M                 // 256
#define CBC_TK BSP_CBC_TILE_K                 // 64
#define CBC_SEG_MAX 4                         // GTiles per segment, at most
#define CBC_UNROLL 8
#define CBC_NMAX 8
#define CBC_WS_COUNTERS 65536                 // bytes of arrival counters at the workspace's start
#define CBC_OOR 0xFFFFFFF0u

template <int NMAX>
__global__ __launch_bounds__(256) void k_cbc_f16(const uint32_t *__restrict__ tile_offsets,
                                                 const uint32_t *__restrict__ colinfo,
                                                 const uint64_t *__restrict__ bitmaps,
                                                 const uint16_t *__restrict__ values, uint32_t values_bytes, int M,
                                                 int K, const uint16_t *__restrict__ X, int N, float tau,
                                                 uint16_t *__restrict__ Y, float *ws_part, uint32_t *ws_cnt, int S,
                                                 int G) {
    __shared__ float xs[NMAX][CBC_SEG_MAX * CBC_TK];
    __shared__ uint16_t list[CBC_SEG_MAX * CBC_TK];
    __shared__ int wcount[4];
    __shared__ int flag;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int gcols = (K + CBC_TK - 1) / CBC_TK;
    const int band = (int)blockIdx.x / S, seg = (int)blockIdx.x % S;
    const int gc0 = seg * G, gc1 = min(gcols, gc0 + G);
    const __amdgpu_buffer_rsrc_t vrs = bsp_rsrc(values, values_bytes);
    const int64_t gbase = (int64_t)band * gcols;
    float acc[NMAX];
#pragma unroll
    for (int n = 0; n < NMAX; ++n) acc[n] = 0.f;

    // the segment in chunks of up to CBC_SEG_MAX GTiles
    for (int cg = gc0; cg < gc1; cg += CBC_SEG_MAX) {
        const int k0 = cg * CBC_TK, k1 = min(K, min(gc1, cg + CBC_SEG_MAX) * CBC_TK);
        const int ncols = max(0, k1 - k0);
        if (cg > gc0) __syncthreads();              // the previous chunk's list and X are read

        // (1) X of the chunk, thresholded; the active columns
        const int t = threadIdx.x;
        bool act = false;
        if (t < ncols) {
#pragma unroll
            for (int n = 0; n < NMAX; ++n) {
                float x = 0.f;
                if (n < N) {
                    x = bsp_h2f(X[(int64_t)n * K + k0 + t]);
                    x = fabsf(x) > tau ? x : 0.f;
                    act = act || x != 0.f;
                }
                xs[n][t] = x;
            }
        }
        const uint64_t bal = __ballot(act);
        if (lane == 0) wcount[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int before = 0, nact = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            before += w < wave ? wcount[w] : 0;
            nact += wcount[w];
        }
        if (act) {
            const uint32_t below =
                    __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            list[before + (int)below] = (uint16_t)t;
        }
        __syncthreads();

        // (2) the active columns, CBC_UNROLL at a time
        for (int i0 = 0; i0 < nact; i0 += CBC_UNROLL) {
            uint32_t vpos[CBC_UNROLL];
            int col[CBC_UNROLL];
#pragma unroll
            for (int u = 0; u < CBC_UNROLL; ++u) {
                const int i = min(i0 + u, nact - 1);
                const int c = __builtin_amdgcn_readfirstlane(list[i]);
                col[u] = c;
                const int k = k0 + c;
                const int64_t g = gbase + (k >> 6);
                const int64_t cc = g * CBC_TK + (k & 63);
                const uint64_t *bw = bitmaps + cc * (CBC_TM / 64);
                const uint64_t w0 = bw[0], w1 = bw[1], w2 = bw[2], w3 = bw[3];
                const uint32_t ci = colinfo[cc];
                const uint32_t to = tile_offsets[g];
                const uint64_t mine = wave == 0 ? w0 : wave == 1 ? w1 : wave == 2 ? w2 : w3;
                const uint32_t prefix = (wave > 0 ? (uint32_t)__builtin_popcountll(w0) : 0u) +
                                        (wave > 1 ? (uint32_t)__builtin_popcountll(w1) : 0u) +
                                        (wave > 2 ? (uint32_t)__builtin_popcountll(w2) : 0u);
                const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mine >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mine, 0u));
                const bool bit = ((mine >> lane) & 1ull) != 0 && i0 + u < nact;
                vpos[u] = bit ? (to + (ci >> 16) + prefix + rank) * 2u : CBC_OOR;
            }
            uint32_t hv[CBC_UNROLL];
#pragma unroll
            for (int u = 0; u < CBC_UNROLL; ++u) hv[u] = __builtin_amdgcn_raw_buffer_load_b16(vrs, vpos[u], 0, 0);
#pragma unroll
            for (int u = 0; u < CBC_UNROLL; ++u) {
                const float w = bsp_h2f((uint16_t)hv[u]);
#pragma unroll
                for (int n = 0; n < NMAX; ++n)
                    if (n < N) acc[n] = fmaf(w, xs[n][col[u]], acc[n]);
            }
        }
    }

    // (3) the band's rows
    const int row = wave * 64 + lane;
    const int m = band * CBC_TM + row;
    if (S == 1) {
        if (m < M)
#pragma unroll
            for (int n = 0; n < NMAX; ++n)
                if (n < N) Y[(int64_t)n * M + m] = bsp_f2h(acc[n]);
        return;
    }
#pragma unroll
    for (int n = 0; n < NMAX; ++n)
        if (n < N) sk_ws_store(ws_part + (((int64_t)band * S + seg) * N + n) * CBC_TM + row, acc[n]);
    __builtin_amdgcn_s_waitcnt(0);           // this thread's partial stores completed
    __syncthreads();
    if (threadIdx.x == 0)
        flag = (int)__hip_atomic_fetch_add(&ws_cnt[band], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (flag != S - 1) return;
    if (m < M)
        for (int n = 0; n < N; ++n) {
            float s = 0.f;
            for (int sp = 0; sp < S; ++sp) s += sk_ws_load(ws_part + (((int64_t)band * S + sp) * N + n) * CBC_TM + row);
            Y[(int64_t)n * M + m] = bsp_f2h(s);
        }
    if (threadIdx.x == 0) sk_ws_store(&ws_cnt[band], 0u);   // ready for the next call
}

struct CbcPlan {
    int bands = 0, S = 1, G = CBC_SEG_MAX;
    int64_t ws_bytes = 0;
};

// Segments per band: enough workgroups to give every CU four (G >= 1
// GTile each), when a workspace is given.
static CbcPlan cbc_plan(int64_t M, int64_t K, int64_t N, bool split) {
    CbcPlan p;
    p.bands = (int)((M + CBC_TM - 1) / CBC_TM);
    const int64_t gcols = (K + CBC_TK - 1) / CBC_TK;
    if (!split || gcols <= 1 || p.bands > CBC_WS_COUNTERS / 4) {
        p.S = 1;
        p.G = (int)std::max<int64_t>(1, gcols);
        return p;
    }
    int64_t G = std::max<int64_t>(1, std::min<int64_t>(CBC_SEG_MAX, (int64_t)p.bands * gcols / (4 * BT_CUS)));
    p.G = (int)G;
    p.S = (int)((gcols + G - 1) / G);
    p.ws_bytes = CBC_WS_COUNTERS + (int64_t)p.bands * p.S * N * CBC_TM * 4;
    return p;
}
