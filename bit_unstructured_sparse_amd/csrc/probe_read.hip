// probe_read.hip -- streaming-read probe: how fast one MI355X (gfx950) can
// read a given number of bytes from HBM in one kernel launch.
//
// This is measurement infrastructure, not part of the SpMM: the benchmark
// reads the SpMM's roofline fraction against the vendor HBM peak, and reports
// beside it what a plain read of the same byte count achieves per launch on
// the same box (and what a read of >= 1 GiB achieves), so that launch ramp-up
// and first-byte latency are visible as a ceiling of their own.
//
// Each thread reads 16-byte granules (64 lanes x 16 B = 1 KB per wavefront
// instruction, fully coalesced), granule g = i * threads + tid, with BSP_PR_U
// loads issued before any is used; the granules are XOR-folded and one dword
// per wavefront goes to `sink` so no load can be dropped. Modes:
//   0  loads into VGPRs, default cache policy
//   1  loads into VGPRs, non-temporal (the policy of the SpMM's weight stream)
//   2  LDS DMA (buffer_load ... lds, 16 B per lane, non-temporal): the SpMM's
//      payload path; each wavefront cycles through 8 KB of LDS of its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsp_probe.h"

#define BSP_PR_U 8        // loads in flight per thread before the first use
#define BSP_PR_LDS_WAVE (8 * 1024)

typedef int pr_v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pr_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int MODE>
__global__ __launch_bounds__(1024) void k_probe_read(const uint8_t *__restrict__ buf, uint32_t bytes,
                                                     uint32_t *__restrict__ sink) {
    extern __shared__ __attribute__((aligned(16))) uint8_t pr_smem[];
    const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t nthreads = gridDim.x * blockDim.x;
    const uint32_t ngran = bytes >> 4;
    const __amdgpu_buffer_rsrc_t rs = pr_rsrc(buf, bytes);
    const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t acc = 0;
    uint32_t slot = 0;
    for (uint32_t g0 = tid; g0 < ngran; g0 += BSP_PR_U * nthreads) {
        if constexpr (MODE == 2) {
#pragma unroll
            for (int u = 0; u < BSP_PR_U; ++u) {
                const uint32_t g = g0 + (uint32_t)u * nthreads;
                // lanes past the end read zeros (out of the buffer's range)
                const uint32_t off = g < ngran ? g * 16u : 0xFFFFFFF0u;
                typedef __attribute__((address_space(3))) void lds_void;
                lds_void *dst = (lds_void *)(pr_smem + wave * BSP_PR_LDS_WAVE + (slot & 7u) * 1024u);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, off, 0, 0, 2);
                ++slot;
            }
        } else {
            pr_v4i v[BSP_PR_U];
#pragma unroll
            for (int u = 0; u < BSP_PR_U; ++u) {
                const uint32_t g = g0 + (uint32_t)u * nthreads;
                const uint32_t off = g < ngran ? g * 16u : 0xFFFFFFF0u;
                v[u] = __builtin_bit_cast(pr_v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, MODE == 1 ? 2 : 0));
            }
#pragma unroll
            for (int u = 0; u < BSP_PR_U; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
        }
    }
    if constexpr (MODE == 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // fold a dword of every KB slot this wavefront wrote
#pragma unroll
        for (int k = 0; k < 8; ++k) acc ^= ((const uint32_t *)(pr_smem + wave * BSP_PR_LDS_WAVE + k * 1024))[lane];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
    if (lane == 0) sink[tid >> 6] = acc;
}

extern "C" int bsp_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int mode, int grid, int block,
                              hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || bytes > (int64_t)UINT32_MAX - 15)
        return 1;
    if (mode < 0 || mode > 2 || grid < 1 || block < 64 || block > 1024 || block % 64 != 0) return 1;
    const size_t lds = mode == 2 ? (size_t)(block / 64) * BSP_PR_LDS_WAVE : 0;
    if (lds > 160 * 1024) return 1;
    switch (mode) {
        case 0:
            hipLaunchKernelGGL(k_probe_read<0>, dim3(grid), dim3(block), 0, stream, (const uint8_t *)buf,
                               (uint32_t)bytes, sink);
            break;
        case 1:
            hipLaunchKernelGGL(k_probe_read<1>, dim3(grid), dim3(block), 0, stream, (const uint8_t *)buf,
                               (uint32_t)bytes, sink);
            break;
        default:
            (void)hipFuncSetAttribute((const void *)k_probe_read<2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)lds);
            hipLaunchKernelGGL(k_probe_read<2>, dim3(grid), dim3(block), lds, stream, (const uint8_t *)buf,
                               (uint32_t)bytes, sink);
            break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int64_t bsp_probe_sink_words(int grid, int block) { return (int64_t)grid * (block / 64); }
