// encode.cpp -- host-side BT64 encoder, int4 activation packer, status strings.
//
// The format is UnionSparse's IE-BME ("UnionSparse: An Index-Efficient
// Sparsity Framework for Low-Bit Sparse LLM Inference on Edge", IEEE TCAD,
// Sec. V-A) with a single area per tile on 1 x 64 row tiles: one 64-bit
// occupancy word per tile (first column = LSB, Fig. 7), a prefix offset per
// tile ("Union Value Offsets" with Q = 1) and the nonzeros packed densely in
// tile order ("Compressed Values"). Encoding is an offline step whose result
// is cached (Sec. V-B), so it runs on the host.
//
// Work split: pass 1 counts nonzeros per row (and range-checks int4 values)
// on all threads; an exclusive scan gives each row's first payload element;
// pass 2 writes each row's words, offsets and payload independently. For
// int4 a row may start in the high nibble of a byte whose low nibble belongs
// to the previous row, so byte writes at block boundaries are merged after
// the threads join: every thread writes only bytes that lie wholly inside its
// own element range and hands its two boundary half-bytes back.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "bitmap_spmm.h"

namespace {

constexpr int64_t kMinRowsPerThread = 64;

inline bool f16_is_zero(uint16_t h) { return (h & 0x7FFFu) == 0; }

int hw_threads() {
    unsigned n = std::thread::hardware_concurrency();
    if (n == 0) n = 1;
    return (int)std::min<unsigned>(n, 64u);
}

// Number of threads used for M rows (deterministic for a given machine).
int plan_threads(int64_t M) {
    int nt = hw_threads();
    int64_t want = (M + kMinRowsPerThread - 1) / kMinRowsPerThread;
    if (want < nt) nt = (int)std::max<int64_t>(want, 1);
    return nt;
}

// Runs fn(thread_index, row_begin, row_end) over plan_threads(M) contiguous row blocks.
template <class F>
void parallel_rows(int64_t M, F &&fn) {
    const int nt = plan_threads(M);
    if (nt <= 1) { fn(0, 0, M); return; }
    std::vector<std::thread> th;
    th.reserve(nt);
    for (int i = 0; i < nt; ++i) {
        int64_t r0 = M * i / nt, r1 = M * (i + 1) / nt;
        th.emplace_back([&fn, i, r0, r1] { fn(i, r0, r1); });
    }
    for (auto &t : th) t.join();
}

struct Boundary {            // int4 half-bytes at the edges of a thread's element range
    int64_t first_byte = -1; // byte index of a leading high nibble (range starts odd)
    uint8_t first_hi = 0;
    int64_t last_byte = -1;  // byte index of a trailing low nibble (range ends odd)
    uint8_t last_lo = 0;
};

}  // namespace

extern "C" int encode_bitmap_tiles(int dtype, const void *W, int64_t M, int64_t K, int64_t ldw,
                                   uint64_t *bitmaps, uint32_t *offsets,
                                   void *payload, int64_t payload_capacity_bytes,
                                   int64_t *nnz_out, int64_t *payload_bytes_out) {
    if (dtype != BSP_INT4 && dtype != BSP_FP16 && dtype != BSP_INT2) return BSP_E_ARG;
    if (M < 0 || K < 0 || ldw < K) return BSP_E_ARG;
    if (M > 0 && K > 0 && W == nullptr) return BSP_E_ARG;
    if (payload_capacity_bytes < 0) return BSP_E_ARG;
    if ((bitmaps == nullptr) != (offsets == nullptr)) return BSP_E_ARG;
    if (payload != nullptr && bitmaps == nullptr) return BSP_E_ARG;
    const int64_t T = (K + 63) / 64;

    // Pass 1: per-row counts and the int4 range check.
    std::vector<int64_t> row_nnz((size_t)M + 1, 0);
    std::atomic<bool> bad_range{false};
    parallel_rows(M, [&](int, int64_t r0, int64_t r1) {
        for (int64_t m = r0; m < r1; ++m) {
            int64_t c = 0;
            if (dtype == BSP_INT4 || dtype == BSP_INT2) {
                const int lo = dtype == BSP_INT4 ? -8 : -2, hi = dtype == BSP_INT4 ? 7 : 1;
                const int8_t *row = (const int8_t *)W + m * ldw;
                for (int64_t k = 0; k < K; ++k) {
                    int v = row[k];
                    if (v < lo || v > hi) { bad_range.store(true, std::memory_order_relaxed); }
                    c += (v != 0);
                }
            } else {
                const uint16_t *row = (const uint16_t *)W + m * ldw;
                for (int64_t k = 0; k < K; ++k) c += !f16_is_zero(row[k]);
            }
            row_nnz[(size_t)m] = c;
        }
    });
    if (bad_range.load()) return BSP_E_RANGE;

    // Exclusive scan: row_start[m] = nonzeros in rows 0..m-1.
    std::vector<int64_t> row_start((size_t)M + 1, 0);
    for (int64_t m = 0; m < M; ++m) row_start[(size_t)m + 1] = row_start[(size_t)m] + row_nnz[(size_t)m];
    const int64_t nnz = row_start[(size_t)M];
    if (nnz > (int64_t)UINT32_MAX) return BSP_E_OVERFLOW;
    const int64_t bytes = dtype == BSP_INT4 ? (nnz + 1) / 2 : dtype == BSP_INT2 ? (nnz + 3) / 4 : 2 * nnz;
    if (nnz_out) *nnz_out = nnz;
    if (payload_bytes_out) *payload_bytes_out = bytes;
    if (payload == nullptr) {
        if (bitmaps == nullptr && offsets == nullptr) return BSP_OK;  // pure size query
    } else if (payload_capacity_bytes < bytes) {
        return BSP_E_CAPACITY;
    }

    // Pass 2: words, offsets and payload, row by row.
    const int used_threads = plan_threads(M);
    std::vector<Boundary> bounds((size_t)used_threads);
    parallel_rows(M, [&](int tid, int64_t r0, int64_t r1) {
        Boundary &bd = bounds[(size_t)tid];
        const int64_t e_begin = row_start[(size_t)r0], e_end = row_start[(size_t)r1];
        uint8_t *p8 = (uint8_t *)payload;
        uint16_t *p16 = (uint16_t *)payload;
        int64_t e = e_begin;
        uint8_t pending = 0;  // low nibble waiting for its partner (int4)
        for (int64_t m = r0; m < r1; ++m) {
            for (int64_t t = 0; t < T; ++t) {
                const int64_t g = m * T + t;
                offsets[g] = (uint32_t)e;
                uint64_t word = 0;
                const int64_t k0 = 64 * t;
                const int jn = (int)std::min<int64_t>(64, K - k0);
                if (dtype == BSP_INT4) {
                    const int8_t *row = (const int8_t *)W + m * ldw + k0;
                    for (int j = 0; j < jn; ++j) {
                        int v = row[j];
                        if (v == 0) continue;
                        word |= (uint64_t)1 << j;
                        if (payload) {
                            uint8_t code = (uint8_t)(v & 0xF);
                            if ((e & 1) == 0) {
                                pending = code;
                            } else if (e - 1 < e_begin) {  // leading high nibble: shared byte
                                bd.first_byte = e >> 1;
                                bd.first_hi = code;
                            } else {
                                p8[e >> 1] = (uint8_t)(pending | (code << 4));
                            }
                        }
                        ++e;
                    }
                } else if (dtype == BSP_INT2) {
                    // words only here; the 2-bit codes are packed after the
                    // threads join (four to a byte, across thread boundaries)
                    const int8_t *row = (const int8_t *)W + m * ldw + k0;
                    for (int j = 0; j < jn; ++j)
                        if (row[j] != 0) {
                            word |= (uint64_t)1 << j;
                            ++e;
                        }
                } else {
                    const uint16_t *row = (const uint16_t *)W + m * ldw + k0;
                    for (int j = 0; j < jn; ++j) {
                        uint16_t h = row[j];
                        if (f16_is_zero(h)) continue;
                        word |= (uint64_t)1 << j;
                        if (payload) p16[e] = h;
                        ++e;
                    }
                }
                bitmaps[g] = word;
            }
        }
        if (dtype == BSP_INT4 && payload && (e_end & 1) && e_end - 1 >= e_begin) {
            bd.last_byte = (e_end - 1) >> 1;   // trailing low nibble: shared byte
            bd.last_lo = pending;
        }
    });
    if (M > 0) offsets[M * T] = (uint32_t)nnz;
    else if (offsets) offsets[0] = 0;

    if (dtype == BSP_INT4 && payload) {
        // Merge the half-bytes at thread boundaries. A byte shared by two
        // ranges gets its low nibble from one and its high nibble from the
        // next; a final odd element leaves the high nibble zero.
        uint8_t *p8 = (uint8_t *)payload;
        std::vector<std::pair<int64_t, uint8_t>> lo, hi;
        for (int i = 0; i < used_threads; ++i) {
            const Boundary &bd = bounds[(size_t)i];
            if (bd.last_byte >= 0) lo.push_back({bd.last_byte, bd.last_lo});
            if (bd.first_byte >= 0) hi.push_back({bd.first_byte, bd.first_hi});
        }
        for (auto &x : lo) p8[x.first] = x.second;                 // high nibble zero for now
        for (auto &x : hi) p8[x.first] = (uint8_t)((p8[x.first] & 0x0F) | (x.second << 4));
    }
    if (dtype == BSP_INT2 && payload && bytes > 0) {
        // element e in byte e >> 2 at bits 2 (e & 3), the lowest first
        uint8_t *p8 = (uint8_t *)payload;
        memset(p8, 0, (size_t)bytes);
        int64_t e = 0;
        for (int64_t m = 0; m < M; ++m) {
            const int8_t *row = (const int8_t *)W + m * ldw;
            for (int64_t k = 0; k < K; ++k)
                if (row[k] != 0) {
                    p8[e >> 2] = (uint8_t)(p8[e >> 2] | ((row[k] & 3) << (2 * (e & 3))));
                    ++e;
                }
        }
    }
    return BSP_OK;
}

extern "C" int pack_int4_activations(const int8_t *X, int64_t N, int64_t K, int64_t ldx, uint8_t *Xp) {
    if (N < 0 || K < 0 || ldx < K) return BSP_E_ARG;
    if (N > 0 && K > 0 && (X == nullptr || Xp == nullptr)) return BSP_E_ARG;
    const int64_t stride = (K + 1) / 2;
    for (int64_t n = 0; n < N; ++n) {
        const int8_t *row = X + n * ldx;
        uint8_t *out = Xp + n * stride;
        for (int64_t k = 0; k < K; ++k) {
            int v = row[k];
            if (v < -8 || v > 7) return BSP_E_RANGE;
        }
        for (int64_t b = 0; b < stride; ++b) {
            uint8_t lo = (uint8_t)(row[2 * b] & 0xF);
            uint8_t hi = (2 * b + 1 < K) ? (uint8_t)(row[2 * b + 1] & 0xF) : 0;
            out[b] = (uint8_t)(lo | (hi << 4));
        }
    }
    return BSP_OK;
}

extern "C" const char *bsp_status_string(int status) {
    switch (status) {
        case BSP_OK: return "ok";
        case BSP_E_ARG: return "invalid argument";
        case BSP_E_RANGE: return "weight outside its type's range (int4 [-8, 7], int2 [-2, 1])";
        case BSP_E_CAPACITY: return "payload buffer too small";
        case BSP_E_OVERFLOW: return "size beyond the supported range";
        case BSP_E_HIP: return "HIP launch error";
        case BSP_E_UNSUPPORTED: return "the forced kernel cannot run this shape";
        default: return "unknown status";
    }
}

extern "C" const char *bsp_version(void) { return "0.1.0"; }
