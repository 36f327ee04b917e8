// encode_union.cpp -- host-side IE-BME encoder with bitmap-aware row
// reordering (UnionSparse, Sec. V-A "IE-BME Representation" and Fig. 7;
// Sec. V-B "Bitmap-Aware Row Reordering", Eq. 3-5, Algorithm 1).
//
// Local tiles (LTs) are 16 x 64, in row-major order over the matrix (a band of
// 16 rows, then the tile column); tiles that run past M or K are padded with
// zeros. An LT is split into ra x ca areas (area q = a * ca + c). Logical
// position (i, j) of the (16/ra) x (64/ca) union mask is set when any area
// has a nonzero there; the mask is packed row-major into 16/(ra*ca) 64-bit
// words, the leftmost position in the lowest bit. Every set position emits
// one value from every area (zeros included) at one compact rank: area q's
// value lands at CV[o_t + q P_t + rank], o_t being the sum of Q P over the
// earlier LTs.
//
// With reordering on, each LT's rows are first grouped into 16/ra groups of
// ra by a subset DP that minimises the number of active logical positions:
// F(S) = min over groups g containing the smallest row of S of
// cost(g) + F(S \ g), cost(g) = number of logical columns in which some row
// of g has a nonzero in one of the ca column areas. Ties go to the first
// group in ascending lexicographic order. The DP is evaluated top-down, so
// only the subsets reachable from the full row set are visited (1597 for
// ra = 2). The permutation concatenates, area row by area row, the p-th row
// of every group; it is stored as its inverse (rowpos: nibble r = reordered
// position of tile row r). Tiles are independent, so they are spread over
// threads.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "bitmap_spmm.h"

namespace {

constexpr int kH = BSP_LT_ROWS;   // 16
constexpr int kW = BSP_LT_COLS;   // 64

bool valid_partition(int ra, int ca) {
    auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
    return pow2(ra) && pow2(ca) && ra <= kH && ca <= kW && ra * ca <= 16;
}

int nthreads_for(int64_t units) {
    unsigned n = std::thread::hardware_concurrency();
    if (n == 0) n = 1;
    n = std::min<unsigned>(n, 64u);
    const int64_t want = std::max<int64_t>(1, units / 256);
    return (int)std::min<int64_t>(n, want);
}

template <class F>
void parallel_for(int64_t n, F &&fn) {
    const int nt = nthreads_for(n);
    if (nt <= 1) { fn(0, 0, n); return; }
    std::vector<std::thread> th;
    for (int i = 0; i < nt; ++i) {
        const int64_t a = n * i / nt, b = n * (i + 1) / nt;
        th.emplace_back([&fn, i, a, b] { fn(i, a, b); });
    }
    for (auto &t : th) t.join();
}

// The nonzero pattern of one LT: bit j of rows[r] = (W[16 b + r][64 c + j] != 0).
struct TileBits {
    uint64_t rows[kH];
};

// Number of logical columns (64/ca of them) a set of rows activates: OR the
// rows, then fold the ca column areas onto one another.
inline int group_cost(uint64_t orbits, int ca) {
    const int w = kW / ca;
    const uint64_t m = w == 64 ? ~0ull : ((1ull << w) - 1ull);
    uint64_t f = 0;
    for (int c = 0; c < ca; ++c) f |= (orbits >> (c * w)) & m;
    return __builtin_popcountll(f);
}

// Top-down subset DP of one tile. The memo arrays are per thread and
// stamped, so nothing is cleared between tiles.
struct Reorderer {
    int ra, ca;
    std::vector<uint32_t> stamp;
    std::vector<uint16_t> best;
    std::vector<uint16_t> choice;
    uint32_t cur = 0;
    const TileBits *tb = nullptr;

    Reorderer(int ra_, int ca_) : ra(ra_), ca(ca_), stamp(1u << kH, 0), best(1u << kH), choice(1u << kH) {}

    int F(uint32_t S) {
        if (S == 0) return 0;
        if (stamp[S] == cur) return best[S];
        int members[kH], n = 0;
        for (int r = 0; r < kH; ++r)
            if ((S >> r) & 1u) members[n++] = r;
        const int r0 = members[0];
        const int k = ra - 1;                       // rows to pick besides r0, from members[1..n)
        int idx[kH];
        for (int i = 0; i < k; ++i) idx[i] = 1 + i;
        int bestv = -1;
        uint32_t bestg = 0;
        for (;;) {
            uint32_t g = 1u << r0;
            uint64_t orbits = tb->rows[r0];
            for (int i = 0; i < k; ++i) {
                g |= 1u << members[idx[i]];
                orbits |= tb->rows[members[idx[i]]];
            }
            const int v = group_cost(orbits, ca) + F(S & ~g);
            if (bestv < 0 || v < bestv) { bestv = v; bestg = g; }
            // next combination in lexicographic order
            int i = k - 1;
            while (i >= 0 && idx[i] == n - k + i) --i;
            if (i < 0) break;
            ++idx[i];
            for (int j = i + 1; j < k; ++j) idx[j] = idx[j - 1] + 1;
        }
        stamp[S] = cur;
        best[S] = (uint16_t)bestv;
        choice[S] = (uint16_t)bestg;
        return bestv;
    }

    // pi[p * G + g] = row p of group g; groups in order of their first row.
    void solve(const TileBits &t, int pi[kH]) {
        tb = &t;
        if (++cur == 0) {                           // stamp wrapped: clear once
            std::fill(stamp.begin(), stamp.end(), 0u);
            cur = 1;
        }
        const uint32_t full = (1u << kH) - 1u;
        F(full);
        const int G = kH / ra;
        int groups[kH][kH];
        int ng = 0;
        for (uint32_t S = full; S != 0;) {
            const uint32_t g = choice[S];
            int p = 0;
            for (int r = 0; r < kH; ++r)
                if ((g >> r) & 1u) groups[ng][p++] = r;
            ++ng;
            S &= ~g;
        }
        // groups come out with ascending first rows and sorted members: the
        // canonical order already
        for (int p = 0; p < ra; ++p)
            for (int g = 0; g < G; ++g) pi[p * G + g] = groups[g][p];
    }
};

void tile_bits(const int8_t *W, int64_t M, int64_t K, int64_t ldw, int64_t b, int64_t c, TileBits *t) {
    for (int r = 0; r < kH; ++r) {
        uint64_t v = 0;
        const int64_t m = b * kH + r;
        if (m < M) {
            const int8_t *row = W + m * ldw + c * kW;
            const int64_t n = std::min<int64_t>(kW, K - c * kW);
            for (int64_t j = 0; j < n; ++j)
                if (row[j] != 0) v |= 1ull << j;
        }
        t->rows[r] = v;
    }
}

// One LT's mask words, its P, and (when vals != nullptr) its Q streams in
// CV order (stream q at vals[q * P ...]).
int tile_encode(const int8_t *W, int64_t M, int64_t K, int64_t ldw, int64_t b, int64_t c, int ra, int ca,
                const int pi[kH], uint64_t *words, int8_t *vals) {
    const int h = kH / ra, w = kW / ca;
    const int nwords = h * w / 64;
    for (int i = 0; i < nwords; ++i) words[i] = 0;
    auto value = [&](int rr, int col) -> int8_t {      // reordered tile row rr, tile column col
        const int64_t m = b * kH + pi[rr];
        const int64_t k = c * kW + col;
        return (m < M && k < K) ? W[m * ldw + k] : (int8_t)0;
    };
    int P = 0;
    for (int i = 0; i < h; ++i)
        for (int j = 0; j < w; ++j) {
            bool any = false;
            for (int a = 0; a < ra && !any; ++a)
                for (int cc = 0; cc < ca && !any; ++cc) any = value(a * h + i, cc * w + j) != 0;
            if (!any) continue;
            const int f = i * w + j;
            words[f >> 6] |= 1ull << (f & 63);
            ++P;
        }
    if (vals != nullptr) {
        int rank = 0;
        for (int i = 0; i < h; ++i)
            for (int j = 0; j < w; ++j) {
                const int f = i * w + j;
                if (!((words[f >> 6] >> (f & 63)) & 1ull)) continue;
                for (int a = 0; a < ra; ++a)
                    for (int cc = 0; cc < ca; ++cc) vals[(a * ca + cc) * P + rank] = value(a * h + i, cc * w + j);
                ++rank;
            }
    }
    return P;
}

uint64_t rowpos_of(const int pi[kH]) {
    uint64_t v = 0;
    for (int p = 0; p < kH; ++p) v |= (uint64_t)p << (4 * pi[p]);
    return v;
}

}  // namespace

extern "C" int64_t union_tile_count(int64_t M, int64_t K) {
    if (M < 0 || K < 0) return -1;
    return ((M + kH - 1) / kH) * ((K + kW - 1) / kW);
}

extern "C" int union_mask_words(int ra, int ca) {
    return valid_partition(ra, ca) ? 16 / (ra * ca) : 0;
}

extern "C" int encode_union_tiles(const int8_t *W, int64_t M, int64_t K, int64_t ldw, int ra, int ca, int reorder,
                                  uint64_t *ubitmaps, uint32_t *offsets, uint64_t *rowpos,
                                  uint8_t *payload, int64_t payload_capacity_bytes,
                                  int64_t *nvals_out, int64_t *payload_bytes_out) {
    if (!valid_partition(ra, ca)) return BSP_E_ARG;
    if (M < 0 || K < 0 || ldw < K || payload_capacity_bytes < 0) return BSP_E_ARG;
    if (M > 0 && K > 0 && W == nullptr) return BSP_E_ARG;
    const bool arrays = ubitmaps != nullptr;
    if ((offsets != nullptr) != arrays || (rowpos != nullptr) != arrays) return BSP_E_ARG;
    if (payload != nullptr && !arrays) return BSP_E_ARG;
    // values must be int4
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            const int v = W[m * ldw + k];
            if (v < -8 || v > 7) return BSP_E_RANGE;
        }
    const int64_t bands = (M + kH - 1) / kH, T = (K + kW - 1) / kW, nlt = bands * T;
    const int Q = ra * ca, nwords = 16 / Q;

    // pass 1: permutation and P of every tile
    std::vector<uint8_t> perms((size_t)nlt * kH);
    std::vector<int64_t> P((size_t)nlt);
    parallel_for(nlt, [&](int, int64_t a, int64_t e) {
        Reorderer R(ra, ca);
        TileBits tb;
        uint64_t words[16];
        int pi[kH];
        for (int64_t t = a; t < e; ++t) {
            const int64_t b = t / (T > 0 ? T : 1), c = t - b * T;
            if (reorder && ra > 1) {
                tile_bits(W, M, K, ldw, b, c, &tb);
                R.solve(tb, pi);
            } else {
                for (int r = 0; r < kH; ++r) pi[r] = r;
            }
            for (int r = 0; r < kH; ++r) perms[(size_t)t * kH + r] = (uint8_t)pi[r];
            P[(size_t)t] = tile_encode(W, M, K, ldw, b, c, ra, ca, pi, words, nullptr);
        }
    });
    std::vector<int64_t> off((size_t)nlt + 1, 0);
    for (int64_t t = 0; t < nlt; ++t) off[(size_t)t + 1] = off[(size_t)t] + (int64_t)Q * P[(size_t)t];
    const int64_t nvals = off[(size_t)nlt];
    const int64_t pbytes = (nvals + 1) / 2;
    if (nvals_out) *nvals_out = nvals;
    if (payload_bytes_out) *payload_bytes_out = pbytes;
    if (nvals > (int64_t)UINT32_MAX) return BSP_E_OVERFLOW;
    if (!arrays) return BSP_OK;
    if (payload != nullptr && payload_capacity_bytes < pbytes) return BSP_E_CAPACITY;
    for (int64_t t = 0; t <= nlt; ++t) offsets[t] = (uint32_t)off[(size_t)t];

    // pass 2: words, rowpos, payload. A tile's values start at an even
    // element (Q even) or anywhere (Q = 1); threads write whole bytes of their
    // own range and hand the half-bytes at its edges back.
    struct Edge {
        int64_t byte = -1;
        uint8_t nib = 0;
        bool high = false;
    };
    const int nt = nthreads_for(nlt);
    std::vector<Edge> edges((size_t)nt * 2);
    if (payload != nullptr && pbytes > 0) memset(payload, 0, (size_t)pbytes);
    parallel_for(nlt, [&](int ti, int64_t a, int64_t e) {
        std::vector<int8_t> vals((size_t)kH * kW);
        int pi[kH];
        for (int64_t t = a; t < e; ++t) {
            const int64_t b = t / (T > 0 ? T : 1), c = t - b * T;
            for (int r = 0; r < kH; ++r) pi[r] = perms[(size_t)t * kH + r];
            rowpos[t] = rowpos_of(pi);
            const int p = tile_encode(W, M, K, ldw, b, c, ra, ca, pi, ubitmaps + t * nwords, vals.data());
            if (payload == nullptr) continue;
            const int64_t e0 = off[(size_t)t], e1 = e0 + (int64_t)Q * p;
            const int64_t lo = off[(size_t)a], hi = off[(size_t)e];
            for (int64_t el = e0; el < e1; ++el) {
                const uint8_t code = (uint8_t)vals[(size_t)(el - e0)] & 0xF;
                const int64_t byte = el >> 1;
                const bool high = el & 1;
                // a byte shared with the neighbouring thread's range
                const bool shared = (high && el == lo) || (!high && el + 1 == hi && el + 1 < nvals);
                if (shared) {
                    Edge &ed = edges[(size_t)ti * 2 + (el == lo ? 0 : 1)];
                    ed.byte = byte;
                    ed.nib = code;
                    ed.high = high;
                    continue;
                }
                payload[byte] = (uint8_t)(payload[byte] | (high ? (code << 4) : code));
            }
        }
    });
    for (const Edge &ed : edges)
        if (ed.byte >= 0) payload[ed.byte] = (uint8_t)(payload[ed.byte] | (ed.high ? (ed.nib << 4) : ed.nib));
    return BSP_OK;
}
