// kernels_rowwave.hip -- the plain kernel: one wavefront per output row.
//
// Lane l walks tiles t = l, l+64, ... of its row. For every set bit j of a
// tile word it takes the payload element offsets[g] + (bits of the word
// below j) -- the masked-popcount rank of SPDP's HAD-SMBD (Sec. 4.2.1) and
// the compact rank of UnionSparse's Compressed Values (Sec. V-A) -- and
// multiplies it with X[64t+j][n] for every n. A wave-wide sum gives Y[n][m].
// It reads every operand through the caches one element at a time, so it is
// the simple baseline the faster kernels are measured against.

// WB: width of a stored weight (4: int4 codes two per byte; 2: int2 codes
// four per byte, the W2A4 variant), low bits first.
template <int NB, int WB = 4>
__global__ __launch_bounds__(256) void k_rowwave_w4a4(const uint64_t *__restrict__ bitmaps,
                                                      const uint32_t *__restrict__ offsets,
                                                      const uint8_t *__restrict__ payload, uint32_t payload_bytes,
                                                      int M, int K, const uint8_t *__restrict__ X, int N,
                                                      int32_t *__restrict__ Y) {
    const int m = blockIdx.x * (blockDim.x / BSP_WAVE) + threadIdx.x / BSP_WAVE;
    const int lane = threadIdx.x % BSP_WAVE;
    if (m >= M) return;
    const int T = (K + 63) / 64;
    const int xs = (K + 1) / 2;
    const __amdgpu_buffer_rsrc_t pr = bsp_rsrc(payload, payload_bytes);
    // X through a bounded resource too: a stray bit past K in a corrupt word
    // then reads zero instead of memory past X.
    const __amdgpu_buffer_rsrc_t xr = bsp_rsrc(X, (uint32_t)(N * xs));
    int acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = 0;
    for (int t = lane; t < T; t += BSP_WAVE) {
        const int64_t g = (int64_t)m * T + t;
        uint64_t word = bitmaps[g];
        uint32_t e = offsets[g];
        while (word) {
            const int j = __builtin_ctzll(word);
            word &= word - 1;
            int w;
            if constexpr (WB == 4) {
                const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(pr, e >> 1, 0, 0);
                w = bsp_sext4(byte >> ((e & 1) * 4));
            } else {
                const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(pr, e >> 2, 0, 0);
                w = (int)((byte >> ((e & 3) * 2)) << 30) >> 30;
            }
            ++e;
            const int k = 64 * t + j;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if (n < N) {
                    const uint32_t xb = __builtin_amdgcn_raw_buffer_load_b8(xr, (uint32_t)(n * xs + (k >> 1)), 0, 0);
                    acc[n] += w * bsp_sext4(xb >> ((k & 1) * 4));
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        if (n < N) {
            const int s = bsp_wave_sum(acc[n]);
            if (lane == 0) Y[(int64_t)n * M + m] = s;
        }
    }
}

template <int NB>
__global__ __launch_bounds__(256) void k_rowwave_f16(const uint64_t *__restrict__ bitmaps,
                                                     const uint32_t *__restrict__ offsets,
                                                     const uint16_t *__restrict__ payload, uint32_t payload_bytes,
                                                     int M, int K, const uint16_t *__restrict__ X, int N,
                                                     uint16_t *__restrict__ Y) {
    const int m = blockIdx.x * (blockDim.x / BSP_WAVE) + threadIdx.x / BSP_WAVE;
    const int lane = threadIdx.x % BSP_WAVE;
    if (m >= M) return;
    const int T = (K + 63) / 64;
    const __amdgpu_buffer_rsrc_t pr = bsp_rsrc(payload, payload_bytes);
    const __amdgpu_buffer_rsrc_t xr = bsp_rsrc(X, (uint32_t)(N * K * 2));
    float acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = 0.f;
    for (int t = lane; t < T; t += BSP_WAVE) {
        const int64_t g = (int64_t)m * T + t;
        uint64_t word = bitmaps[g];
        uint32_t e = offsets[g];
        while (word) {
            const int j = __builtin_ctzll(word);
            word &= word - 1;
            const uint16_t wb = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(pr, e * 2u, 0, 0);
            const float w = bsp_h2f(wb);
            ++e;
            const int k = 64 * t + j;
#pragma unroll
            for (int n = 0; n < NB; ++n)
                if (n < N) {
                    const uint16_t xh = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(xr, (uint32_t)(n * K + k) * 2u, 0, 0);
                    acc[n] = fmaf(w, bsp_h2f(xh), acc[n]);
                }
        }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        if (n < N) {
            const float s = bsp_wave_sum(acc[n]);
            if (lane == 0) Y[(int64_t)n * M + m] = bsp_f2h(s);
        }
    }
}

template <int WB = 4>
static void launch_rowwave_w4a4(const uint64_t *bitmaps, const uint32_t *offsets, const uint8_t *payload,
                                uint32_t payload_bytes, int M, int K, const uint8_t *X, int N, int32_t *Y,
                                hipStream_t stream) {
    const dim3 block(256), grid((unsigned)((M + 3) / 4));
    if (N <= 8)
        hipLaunchKernelGGL((k_rowwave_w4a4<8, WB>), grid, block, 0, stream, bitmaps, offsets, payload, payload_bytes, M, K,
                           X, N, Y);
    else
        hipLaunchKernelGGL((k_rowwave_w4a4<32, WB>), grid, block, 0, stream, bitmaps, offsets, payload, payload_bytes, M,
                           K, X, N, Y);
}

static void launch_rowwave_f16(const uint64_t *bitmaps, const uint32_t *offsets, const uint16_t *payload,
                               uint32_t payload_bytes, int M, int K, const uint16_t *X, int N, uint16_t *Y,
                               hipStream_t stream) {
    const dim3 block(256), grid((unsigned)((M + 3) / 4));
    if (N <= 8)
        hipLaunchKernelGGL(k_rowwave_f16<8>, grid, block, 0, stream, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y);
    else
        hipLaunchKernelGGL(k_rowwave_f16<32>, grid, block, 0, stream, bitmaps, offsets, payload, payload_bytes, M, K, X, N, Y);
}
