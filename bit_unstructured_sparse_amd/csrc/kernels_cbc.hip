// kernels_cbc.hip -- fp16 decode-phase product with dynamic activation
// pruning over the Tiled-CBC format on gfx950: SPDP, Sec. 4.1 (Tiled-CBC)
// and Sec. 4.2 (the spMspV kernel and its HAD-SMBD decoding).
//
// Y[n][m] = sum over k of W[m][k] * x'[n][k], x' = x where |x| > tau, else 0.
// A column k whose activations are all pruned is skipped: its values are
// never read, which is where dynamic pruning saves bytes.
//
// Work split. Rows go in bands of 256 (one column tile of a GTile); a
// workgroup of 16 wavefronts takes one band and a segment of G consecutive
// GTiles: its 4 column groups of 4 wavefronts take GTiles of the segment in
// turn, and wavefront r of a group owns rows 64 r .. 64 r + 63 of the band,
// one per lane (the column-major, CUDA-core style register layout of
// HAD-SMBD: one output row per thread, one column at a time). The groups'
// partials are added in LDS, in group order.
//
// A wavefront takes its quarter of a GTile in two memory round trips, with
// no LDS and no barrier: (1) lane c loads column c's ColInfo, its four
// bitmap words and its N activations (the threshold applied), and the
// wavefront keeps, in lane c, the column's word for its own 64 rows and the
// position of that word's first value (GTile offset + column offset + the
// set bits of the words above); a ballot marks the columns that are active
// and hold a nonzero in these rows (the others are skipped, values unread);
// (2) the listed columns' words, positions and activations are moved to the
// first lanes in column order (one ds_permute per field); for up to 32 of
// them at a time the wavefront reads each column's word and position out of
// its lane (readlane with a constant lane number: uniform values), and
// every lane finds its rank with v_mbcnt and gathers its value (the word
// itself, as a lane mask, sends a lane whose bit is clear past the buffer's
// range, where it reads zero); then it accumulates value x x' in fp32 (x'
// read out of its lane at N = 1, else from a per-wavefront LDS copy of the
// GTile's activations, a broadcast read). A column costs a wavefront about
// nine vector instructions and no scalar ones.
//
// Segments of one band meet through a workspace: each workgroup posts its
// fp32 partials, and the last of the band's workgroups to arrive (an
// agent-scope counter) adds the segments in segment order (so the result
// does not depend on timing) and writes Y in fp16 (round to nearest even).
// Without a workspace one workgroup covers the whole band, CBC_GROUPS
// GTiles at a time.

#define CBC_TM BSP_CBC_TILE_M                 // 256
#define CBC_TK BSP_CBC_TILE_K                 // 64
#define CBC_GROUPS 4                          // column groups per workgroup, one GTile each at a time
#define CBC_UNROLL 32                         // columns whose gathers are in flight at once
#define CBC_NMAX 8
#define CBC_WS_COUNTERS 65536                 // bytes of arrival counters at the workspace's start
#define CBC_OOR 0xFFFFFFF0u

// Lane l of the result is a where bit l of the uniform mask m is set, else b.
__device__ __forceinline__ uint32_t cbc_lane_select(uint64_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(m));
    return r;
}

template <int NMAX>
__global__ __launch_bounds__(1024) void k_cbc_f16(const uint32_t *__restrict__ tile_offsets,
                                                  const uint32_t *__restrict__ colinfo,
                                                  const uint64_t *__restrict__ bitmaps,
                                                  const uint16_t *__restrict__ values, uint32_t values_bytes, int M,
                                                  int K, const uint16_t *__restrict__ X, int N, float tau,
                                                  uint16_t *__restrict__ Y, float *ws_part, uint32_t *ws_cnt, int S,
                                                  int G) {
    __shared__ float part[CBC_GROUPS][NMAX][CBC_TM];
    // per wavefront: x' of the GTile's columns (a column's N values together,
    // read with 16-byte broadcasts), then a zero column
    __shared__ __attribute__((aligned(16))) float xsw[CBC_GROUPS * 4][CBC_TK + 1][NMAX];
    __shared__ int flag;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int rq = wave & 3, grp = wave >> 2;              // row quarter, column group
    const int gcols = (K + CBC_TK - 1) / CBC_TK;
    const int band = (int)blockIdx.x / S, seg = (int)blockIdx.x % S;
    const int gc0 = seg * G, gc1 = min(gcols, gc0 + G);
    const __amdgpu_buffer_rsrc_t vrs = bsp_rsrc(values, values_bytes);
    const int64_t gbase = (int64_t)band * gcols;
    float acc[NMAX];
#pragma unroll
    for (int n = 0; n < NMAX; ++n) acc[n] = 0.f;

    // group grp takes GTiles gc0 + grp, gc0 + grp + CBC_GROUPS, ...
    for (int gcol = gc0 + grp; gcol < gc1; gcol += CBC_GROUPS) {
        const int k = gcol * CBC_TK + lane;
        const int64_t g = gbase + gcol;
        // (1) lane = column of the GTile
        uint64_t mine = 0;
        uint32_t pos = 0;
        float xv[NMAX];
        bool act = false;
#pragma unroll
        for (int n = 0; n < NMAX; ++n) xv[n] = 0.f;
        if (k < K) {
            const uint64_t *bw = bitmaps + (g * CBC_TK + lane) * (CBC_TM / 64);
            const uint64_t w0 = bw[0], w1 = bw[1], w2 = bw[2], w3 = bw[3];
            const uint32_t ci = colinfo[g * CBC_TK + lane];
            const uint32_t to = tile_offsets[g];
#pragma unroll
            for (int n = 0; n < NMAX; ++n)
                if (n < N) {
                    const float x = bsp_h2f(X[(int64_t)n * K + k]);
                    xv[n] = fabsf(x) > tau ? x : 0.f;
                    act = act || xv[n] != 0.f;
                }
            mine = rq == 0 ? w0 : rq == 1 ? w1 : rq == 2 ? w2 : w3;
            pos = to + (ci >> 16) + (rq > 0 ? (uint32_t)__builtin_popcountll(w0) : 0u) +
                  (rq > 1 ? (uint32_t)__builtin_popcountll(w1) : 0u) +
                  (rq > 2 ? (uint32_t)__builtin_popcountll(w2) : 0u);
        }
        const bool listed = act && mine != 0;
        const uint64_t todo = __ballot(listed);
        const int cnt = __builtin_popcountll(todo);
#pragma unroll
        for (int n = 0; n < NMAX; ++n) {
            xsw[wave][lane][n] = xv[n];
            if (lane == 0) xsw[wave][CBC_TK][n] = 0.f;
        }
        // the listed columns' words, value positions and activations (or
        // column numbers) to lanes 0 .. cnt - 1 in column order, the other
        // columns after them: one forward permute per field, so that the
        // column loop reads them with constant lane numbers
        const uint32_t r1 = __builtin_amdgcn_mbcnt_hi((uint32_t)(todo >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)todo, 0u));
        const uint32_t r0 = (uint32_t)lane - r1;
        const int dst = (int)((listed ? r1 : (uint32_t)cnt + r0) * 4u);
        // every lane takes part in each permute (a lane left out would not
        // deliver its column): the results are pinned before the selects so
        // that the compiler cannot move a permute under the selects' mask
        uint32_t tlo = (uint32_t)__builtin_amdgcn_ds_permute(dst, (int)(uint32_t)mine);
        uint32_t thi = (uint32_t)__builtin_amdgcn_ds_permute(dst, (int)(uint32_t)(mine >> 32));
        uint32_t cpos = (uint32_t)__builtin_amdgcn_ds_permute(dst, (int)pos);
        int tx = __builtin_amdgcn_ds_permute(dst, NMAX == 1 ? __float_as_int(xv[0]) : lane);
        asm volatile("" : "+v"(tlo), "+v"(thi), "+v"(cpos), "+v"(tx));
        const bool valid = lane < cnt;
        const uint32_t cmlo = valid ? tlo : 0u, cmhi = valid ? thi : 0u;
        const float cx = valid ? __int_as_float(tx) : 0.f;   // N = 1: the activation
        const int ccol = valid ? tx : CBC_TK;                 // N > 1: the column
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // (2) CBC_UNROLL columns' gathers in flight at a time; a lane past
        // cnt holds an empty word and a zero activation
#pragma unroll
        for (int bt = 0; bt < CBC_TK / CBC_UNROLL; ++bt) {
            if (bt * CBC_UNROLL >= cnt) break;
            uint32_t hv[CBC_UNROLL];
#pragma unroll
            for (int u = 0; u < CBC_UNROLL; ++u) {
                const int j = bt * CBC_UNROLL + u;
                const uint64_t w = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)cmhi, j) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)cmlo, j);
                const uint32_t p = (uint32_t)__builtin_amdgcn_readlane((int)cpos, j);
                const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(w >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)w, 0u));
                const uint32_t vpos = cbc_lane_select(w, (p + rank) * 2u, CBC_OOR);
                hv[u] = __builtin_amdgcn_raw_buffer_load_b16(vrs, vpos, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < CBC_UNROLL; ++u) {
                const int j = bt * CBC_UNROLL + u;
                const float w = bsp_h2f((uint16_t)hv[u]);
                if constexpr (NMAX == 1) {
                    acc[0] = fmaf(w, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cx), j)), acc[0]);
                } else {
                    const int c = __builtin_amdgcn_readlane(ccol, j);
                    if constexpr (NMAX % 4 == 0) {
#pragma unroll
                        for (int n = 0; n < NMAX; n += 4) {
                            const float4 x4 = *reinterpret_cast<const float4 *>(&xsw[wave][c][n]);
                            acc[n] = fmaf(w, x4.x, acc[n]);
                            acc[n + 1] = fmaf(w, x4.y, acc[n + 1]);
                            acc[n + 2] = fmaf(w, x4.z, acc[n + 2]);
                            acc[n + 3] = fmaf(w, x4.w, acc[n + 3]);
                        }
                    } else {
                        static_assert(NMAX == 2, "activation widths 1, 2 or a multiple of 4");
                        const float2 x2 = *reinterpret_cast<const float2 *>(&xsw[wave][c][0]);
                        acc[0] = fmaf(w, x2.x, acc[0]);
                        acc[1] = fmaf(w, x2.y, acc[1]);
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();                    // xsw is read before the next GTile writes it
    }

    // the column groups' partials, added in group order by column group 0's
    // 256 threads (the other wavefronts only take part in the barriers)
    const int row = rq * 64 + lane;
    const bool lead = grp == 0;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) part[grp][n][row] = acc[n];
    __syncthreads();
    if (lead) {
#pragma unroll
        for (int n = 0; n < NMAX; ++n) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < CBC_GROUPS; ++q) v += part[q][n][row];
            acc[n] = v;
        }
    }
    const int m = band * CBC_TM + row;
    if (S == 1) {
        if (lead && m < M)
#pragma unroll
            for (int n = 0; n < NMAX; ++n)
                if (n < N) Y[(int64_t)n * M + m] = bsp_f2h(acc[n]);
        return;
    }
    if (lead)
#pragma unroll
        for (int n = 0; n < NMAX; ++n)
            if (n < N) sk_ws_store(ws_part + (((int64_t)band * S + seg) * N + n) * CBC_TM + row, acc[n]);
    __builtin_amdgcn_s_waitcnt(0);           // this thread's partial stores completed
    __syncthreads();
    if (threadIdx.x == 0)
        flag = (int)__hip_atomic_fetch_add(&ws_cnt[band], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (flag != S - 1) return;
    // the segments' partials, added in segment order; 16 loads in flight at
    // a time (one after the other, each would wait for the one before)
    if (lead && m < M)
        for (int n = 0; n < N; ++n) {
            const float *pp = ws_part + ((int64_t)band * S * N + n) * CBC_TM + row;
            const int64_t stride = (int64_t)N * CBC_TM;
            float s = 0.f;
            for (int s0 = 0; s0 < S; s0 += 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = s0 + u < S ? sk_ws_load(pp + (s0 + u) * stride) : 0.f;
#pragma unroll
                for (int u = 0; u < 16; ++u) s += v[u];
            }
            Y[(int64_t)n * M + m] = bsp_f2h(s);
        }
    if (threadIdx.x == 0) sk_ws_store(&ws_cnt[band], 0u);   // ready for the next call
}

struct CbcPlan {
    int bands = 0, S = 1, G = CBC_GROUPS;
    int64_t ws_bytes = 0;
};

// With a workspace a workgroup takes CBC_GROUPS GTiles of its band (one per
// column group) and the band's segments meet in the workspace; without one
// it takes the whole band.
static CbcPlan cbc_plan(int64_t M, int64_t K, int64_t N, bool split) {
    CbcPlan p;
    p.bands = (int)((M + CBC_TM - 1) / CBC_TM);
    const int64_t gcols = (K + CBC_TK - 1) / CBC_TK;
    if (!split || gcols <= CBC_GROUPS || p.bands > CBC_WS_COUNTERS / 4) {
        p.S = 1;
        p.G = (int)std::max<int64_t>(1, gcols);
        return p;
    }
    p.G = CBC_GROUPS;
    p.S = (int)((gcols + CBC_GROUPS - 1) / CBC_GROUPS);
    p.ws_bytes = CBC_WS_COUNTERS + (int64_t)p.bands * p.S * N * CBC_TM * 4;
    return p;
}
