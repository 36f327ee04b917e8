// encode_cbc.cpp -- host-side Tiled-CBC encoder (SPDP, "Unified Static-Dynamic
// Pruning for Efficient LLM Inference", Sec. 4.1 and Fig. 4(a)).
//
// GTiles of 256 x 64 in row-major order over the matrix (zero-padded past M
// and K). Inside a GTile, column c is a 256 x 1 column tile: four 64-bit
// bitmap words (bit j of word w = row 64 w + j), and its nonzeros in row
// order; the columns follow one another, so a GTile's values are in
// column-major order. TileOffset[g] is GTile g's first value (N_GT + 1
// entries); ColInfo[g][c] = (first value of column c inside the GTile << 16)
// | (nonzeros of column c). fp16 +0 and -0 are zero. GTiles are independent,
// so they are counted and then written on all threads.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "bitmap_spmm.h"

namespace {

constexpr int kTM = BSP_CBC_TILE_M;
constexpr int kTK = BSP_CBC_TILE_K;

template <class F>
void cbc_parallel(int64_t n, F &&fn) {
    unsigned hw = std::thread::hardware_concurrency();
    const int nt = (int)std::max<int64_t>(1, std::min<int64_t>(std::min<unsigned>(hw ? hw : 1, 64u), n / 64));
    if (nt <= 1) { fn(0, n); return; }
    std::vector<std::thread> th;
    for (int i = 0; i < nt; ++i) th.emplace_back([&fn, i, nt, n] { fn(n * i / nt, n * (i + 1) / nt); });
    for (auto &t : th) t.join();
}

inline bool f16_nonzero(uint16_t h) { return (h & 0x7FFFu) != 0; }

}  // namespace

extern "C" int64_t cbc_gtile_count(int64_t M, int64_t K) {
    if (M < 0 || K < 0) return -1;
    return ((M + kTM - 1) / kTM) * ((K + kTK - 1) / kTK);
}

extern "C" int encode_cbc_f16(const uint16_t *W, int64_t M, int64_t K, int64_t ldw, uint32_t *tile_offsets,
                              uint32_t *colinfo, uint64_t *bitmaps, uint16_t *values, int64_t values_capacity,
                              int64_t *nnz_out) {
    if (M < 0 || K < 0 || ldw < K || values_capacity < 0) return BSP_E_ARG;
    if (M > 0 && K > 0 && W == nullptr) return BSP_E_ARG;
    const bool arrays = tile_offsets != nullptr;
    if ((colinfo != nullptr) != arrays || (bitmaps != nullptr) != arrays) return BSP_E_ARG;
    if (values != nullptr && !arrays) return BSP_E_ARG;
    const int64_t gr = (M + kTM - 1) / kTM, gc = (K + kTK - 1) / kTK, ngt = gr * gc;
    std::vector<int64_t> cnt((size_t)ngt, 0);
    cbc_parallel(ngt, [&](int64_t a, int64_t b) {
        for (int64_t g = a; g < b; ++g) {
            const int64_t m0 = (g / gc) * kTM, k0 = (g % gc) * kTK;
            int64_t c = 0;
            for (int64_t m = m0; m < std::min(M, m0 + kTM); ++m)
                for (int64_t k = k0; k < std::min(K, k0 + kTK); ++k) c += f16_nonzero(W[m * ldw + k]);
            cnt[(size_t)g] = c;
        }
    });
    std::vector<int64_t> off((size_t)ngt + 1, 0);
    for (int64_t g = 0; g < ngt; ++g) off[(size_t)g + 1] = off[(size_t)g] + cnt[(size_t)g];
    const int64_t nnz = off[(size_t)ngt];
    if (nnz_out) *nnz_out = nnz;
    if (nnz > (int64_t)UINT32_MAX) return BSP_E_OVERFLOW;
    if (!arrays) return BSP_OK;
    if (values != nullptr && values_capacity < nnz) return BSP_E_CAPACITY;
    for (int64_t g = 0; g <= ngt; ++g) tile_offsets[g] = (uint32_t)off[(size_t)g];
    cbc_parallel(ngt, [&](int64_t a, int64_t b) {
        for (int64_t g = a; g < b; ++g) {
            const int64_t m0 = (g / gc) * kTM, k0 = (g % gc) * kTK;
            int64_t e = off[(size_t)g];
            uint32_t inside = 0;
            for (int c = 0; c < kTK; ++c) {
                const int64_t k = k0 + c;
                uint64_t words[kTM / 64] = {};
                uint32_t n = 0;
                for (int r = 0; r < kTM; ++r) {
                    const int64_t m = m0 + r;
                    if (m >= M || k >= K) continue;
                    const uint16_t h = W[m * ldw + k];
                    if (!f16_nonzero(h)) continue;
                    words[r / 64] |= (uint64_t)1 << (r % 64);
                    if (values) values[e] = h;
                    ++e;
                    ++n;
                }
                for (int w = 0; w < kTM / 64; ++w) bitmaps[(g * kTK + c) * (kTM / 64) + w] = words[w];
                colinfo[g * kTK + c] = (inside << 16) | n;
                inside += n;
            }
        }
    });
    return BSP_OK;
}
