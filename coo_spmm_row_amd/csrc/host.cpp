// host.cpp -- host-side parts of libsnack_coo: the row-sorted COO builder, the
// prune-and-regrow topology update and the error channel.
//
// Builder: Appendix B (Table 7) of the SNACK paper defines the COO triple, the
// CSR index pointer and the CSC view; Section 3.1 notes the formats are
// interchangeable.  The sort here is two stable counting sorts (by column,
// then by row), O(nnz + O + I), and the column view is one more stable
// counting sort of the row-sorted order by column.
//
// Topology update: Appendix G prunes the smallest-magnitude stored entries and
// regrows as many unique positions with the uniform initializer of Algorithm 2
// (draw a row, draw a column, reject pairs already in the live set S).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/snack_coo.h"
#include "internal.h"

namespace snack {

static thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return SNACK_OK;
}

namespace {

constexpr int64_t kInt32Max = 2147483647LL;

// Stable counting sort of `in` (positions) by key(pos) in [0, nkeys).
template <class KeyFn>
void counting_sort(const std::vector<int32_t> &in, std::vector<int32_t> &out, int64_t nkeys,
                   std::vector<int64_t> &count, KeyFn key) {
    count.assign(static_cast<size_t>(nkeys) + 1, 0);
    for (int32_t p : in) ++count[static_cast<size_t>(key(p)) + 1];
    for (int64_t i = 0; i < nkeys; ++i) count[i + 1] += count[i];
    out.resize(in.size());
    for (int32_t p : in) out[static_cast<size_t>(count[key(p)]++)] = p;
}

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): a Weyl sequence with step
// 0x9E3779B97F4A7C15 passed through a variant of the MurmurHash3 finalizer.
struct SplitMix64 {
    uint64_t state;
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ULL;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
        return z ^ (z >> 31);
    }
    // Algorithm 2's getrand(n): multiply-high range reduction into [0, n).
    int64_t below(int64_t n) {
        return static_cast<int64_t>((static_cast<unsigned __int128>(next()) *
                                     static_cast<uint64_t>(n)) >> 64);
    }
};

}  // namespace
}  // namespace snack

using namespace snack;

extern "C" const char *snack_last_error(void) { return g_last_error.c_str(); }

extern "C" int snack_coo_abi_version(void) { return 10; }

namespace snack {
namespace {
constexpr int kNumOptions = 5;
std::atomic<int64_t> g_options[kNumOptions] = {{-1}, {-1}, {-1}, {-1}, {-1}};
}  // namespace

int64_t option(int which) {
    return which >= 0 && which < kNumOptions ? g_options[which].load(std::memory_order_relaxed) : -1;
}
}  // namespace snack

extern "C" int snack_coo_set_option(int opt, int64_t value) {
    if (opt < 0 || opt >= kNumOptions) return fail(SNACK_ERR_DTYPE, "set_option: unknown option %d", opt);
    bool okv = value == -1;
    switch (opt) {
        case SNACK_OPT_TILE: okv = okv || value == 0; break;
        case SNACK_OPT_BWD_FORM: okv = okv || (value >= 0 && value <= 2); break;
        case SNACK_OPT_BAND_MIN_NNZ: okv = okv || value >= 0; break;
        case SNACK_OPT_TOPOLOGY_DRAW_BATCH: okv = okv || value >= 1; break;
        case SNACK_OPT_BF16_DW_MFMA: okv = okv || value == 0 || value == 1; break;
    }
    if (!okv) return fail(SNACK_ERR_SHAPE, "set_option: value %lld out of range for option %d", (long long)value, opt);
    g_options[opt].store(value, std::memory_order_relaxed);
    return ok();
}

extern "C" int64_t snack_coo_get_option(int opt) { return option(opt); }

extern "C" int snack_coo_build(int64_t O, int64_t I, int64_t nnz,
                               const int32_t *rows, const int32_t *cols, const float *vals,
                               int32_t *rows_out, int32_t *cols_out, float *vals_out,
                               int32_t *perm_out, int32_t *row_offsets_out,
                               int32_t *col_perm_out, int32_t *col_rows_out, int32_t *col_cols_out,
                               int32_t *col_offsets_out) {
    try {
        if (O < 0 || I < 0 || nnz < 0 || O > kInt32Max || I > kInt32Max || nnz > kInt32Max)
            return fail(SNACK_ERR_SHAPE, "build: sizes out of range (O=%lld I=%lld nnz=%lld)",
                        (long long)O, (long long)I, (long long)nnz);
        if (nnz > O * I)
            return fail(SNACK_ERR_SHAPE, "build: nnz=%lld exceeds O*I=%lld", (long long)nnz,
                        (long long)(O * I));
        if (nnz > 0 && (!rows || !cols || !rows_out || !cols_out))
            return fail(SNACK_ERR_NULL, "build: rows, cols, rows_out and cols_out are required");
        if (nnz > 0 && vals_out && !vals)
            return fail(SNACK_ERR_NULL, "build: vals_out given without vals");
        for (int64_t k = 0; k < nnz; ++k) {
            if (rows[k] < 0 || rows[k] >= O || cols[k] < 0 || cols[k] >= I)
                return fail(SNACK_ERR_INDEX, "build: entry %lld = (%d, %d) outside %lld x %lld",
                            (long long)k, rows[k], cols[k], (long long)O, (long long)I);
        }
        std::vector<int32_t> ident(static_cast<size_t>(nnz)), by_col, order;
        for (int64_t k = 0; k < nnz; ++k) ident[k] = static_cast<int32_t>(k);
        std::vector<int64_t> count;
        counting_sort(ident, by_col, I, count, [&](int32_t p) { return cols[p]; });
        counting_sort(by_col, order, O, count, [&](int32_t p) { return rows[p]; });
        for (int64_t k = 1; k < nnz; ++k) {
            const int32_t a = order[k - 1], b = order[k];
            if (rows[a] == rows[b] && cols[a] == cols[b])
                return fail(SNACK_ERR_DUPLICATE, "build: (%d, %d) appears at input positions %d and %d",
                            rows[b], cols[b], a, b);
        }
        for (int64_t k = 0; k < nnz; ++k) {
            const int32_t src = order[k];
            rows_out[k] = rows[src];
            cols_out[k] = cols[src];
            if (vals_out) std::memcpy(&vals_out[k], &vals[src], sizeof(float));
            if (perm_out) perm_out[k] = src;
        }
        if (row_offsets_out) {
            // `count` holds the row histogram prefix of the last pass, shifted by the
            // scatter; rebuild it from the sorted rows for clarity.
            std::fill(row_offsets_out, row_offsets_out + O + 1, 0);
            for (int64_t k = 0; k < nnz; ++k) ++row_offsets_out[rows[order[k]] + 1];
            for (int64_t r = 0; r < O; ++r) row_offsets_out[r + 1] += row_offsets_out[r];
        }
        if (col_perm_out || col_rows_out || col_cols_out || col_offsets_out) {
            std::vector<int32_t> sorted_pos(static_cast<size_t>(nnz)), cview;
            for (int64_t k = 0; k < nnz; ++k) sorted_pos[k] = static_cast<int32_t>(k);
            // key of sorted position k is the column of order[k]; stability keeps rows ascending
            counting_sort(sorted_pos, cview, I, count, [&](int32_t k) { return cols[order[k]]; });
            for (int64_t j = 0; j < nnz; ++j) {
                const int32_t k = cview[j];
                if (col_perm_out) col_perm_out[j] = k;
                if (col_rows_out) col_rows_out[j] = rows[order[k]];
                if (col_cols_out) col_cols_out[j] = cols[order[k]];
            }
            if (col_offsets_out) {
                std::fill(col_offsets_out, col_offsets_out + I + 1, 0);
                for (int64_t k = 0; k < nnz; ++k) ++col_offsets_out[cols[k] + 1];
                for (int64_t c = 0; c < I; ++c) col_offsets_out[c + 1] += col_offsets_out[c];
            }
        }
        return ok();
    } catch (const std::bad_alloc &) {
        return fail(SNACK_ERR_NOMEM, "build: out of host memory");
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "build: unexpected exception");
    }
}

extern "C" int snack_coo_init_uniform(int64_t O, int64_t I, int64_t nnz, uint64_t seed, int32_t *rows_out,
                                      int32_t *cols_out, int32_t *row_offsets_out, int64_t *trials_out) {
    try {
        if (O <= 0 || I <= 0 || nnz < 0 || O > kInt32Max || I > kInt32Max || nnz > kInt32Max || nnz > O * I)
            return fail(SNACK_ERR_SHAPE, "init_uniform: bad sizes (O=%lld I=%lld nnz=%lld)", (long long)O,
                        (long long)I, (long long)nnz);
        const uint64_t cells = static_cast<uint64_t>(O) * static_cast<uint64_t>(I);
        if (cells > (1ULL << 34))
            return fail(SNACK_ERR_SHAPE, "init_uniform: O*I=%llu exceeds the 2^34 bitmap limit",
                        (unsigned long long)cells);
        if (nnz > 0 && (!rows_out || !cols_out)) return fail(SNACK_ERR_NULL, "init_uniform: null array");
        // Algorithm 2 from an empty set: rejection against a bitmap of the drawn positions
        std::vector<uint64_t> drawn(static_cast<size_t>((cells + 63) / 64), 0);
        SplitMix64 rng{seed};
        int64_t trials = 0, count = 0;
        while (count < nnz) {
            const int64_t i = rng.below(O);
            const int64_t j = rng.below(I);
            ++trials;
            const uint64_t q = static_cast<uint64_t>(i) * I + j;
            uint64_t &w = drawn[q >> 6];
            const uint64_t bit = 1ULL << (q & 63);
            if (w & bit) continue;
            w |= bit;
            ++count;
        }
        // the bitmap holds exactly the drawn set: reading it in order gives the (row, col) sort
        int64_t at = 0;
        for (size_t wi = 0; wi < drawn.size() && at < nnz; ++wi) {
            for (uint64_t w = drawn[wi]; w; w &= w - 1) {
                const uint64_t q = (static_cast<uint64_t>(wi) << 6) + static_cast<uint64_t>(__builtin_ctzll(w));
                rows_out[at] = static_cast<int32_t>(q / I);
                cols_out[at] = static_cast<int32_t>(q % I);
                ++at;
            }
        }
        if (at != nnz) return fail(SNACK_ERR_INTERNAL, "init_uniform: produced %lld entries", (long long)at);
        if (row_offsets_out) {
            std::fill(row_offsets_out, row_offsets_out + O + 1, 0);
            for (int64_t k = 0; k < nnz; ++k) ++row_offsets_out[rows_out[k] + 1];
            for (int64_t r = 0; r < O; ++r) row_offsets_out[r + 1] += row_offsets_out[r];
        }
        if (trials_out) *trials_out = trials;
        return ok();
    } catch (const std::bad_alloc &) {
        return fail(SNACK_ERR_NOMEM, "init_uniform: out of host memory");
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "init_uniform: unexpected exception");
    }
}

extern "C" int snack_coo_topology_update(int64_t O, int64_t I, int64_t nnz,
                                         const int32_t *rows, const int32_t *cols, const float *vals,
                                         int64_t n_prune, uint64_t seed,
                                         int32_t *rows_out, int32_t *cols_out, float *vals_out,
                                         int32_t *row_offsets_out, int64_t *trials_out) {
    try {
        if (O <= 0 || I <= 0 || nnz < 0 || O > kInt32Max || I > kInt32Max || nnz > kInt32Max ||
            nnz > O * I || n_prune < 0 || n_prune > nnz)
            return fail(SNACK_ERR_SHAPE, "topology: bad sizes (O=%lld I=%lld nnz=%lld n_prune=%lld)",
                        (long long)O, (long long)I, (long long)nnz, (long long)n_prune);
        const uint64_t cells = static_cast<uint64_t>(O) * static_cast<uint64_t>(I);
        if (cells > (1ULL << 34))
            return fail(SNACK_ERR_SHAPE, "topology: O*I=%llu exceeds the 2^34 bitmap limit",
                        (unsigned long long)cells);
        if (nnz > 0 && (!rows || !cols || !vals || !rows_out || !cols_out || !vals_out))
            return fail(SNACK_ERR_NULL, "topology: null array");
        for (int64_t k = 0; k < nnz; ++k) {
            if (rows[k] < 0 || rows[k] >= O || cols[k] < 0 || cols[k] >= I)
                return fail(SNACK_ERR_INDEX, "topology: entry %lld out of range", (long long)k);
            if (k > 0 && (rows[k] < rows[k - 1] || (rows[k] == rows[k - 1] && cols[k] <= cols[k - 1])))
                return fail(SNACK_ERR_UNSORTED, "topology: entry %lld breaks (row, col) order", (long long)k);
        }
        // 1. prune: the n_prune smallest by (|v|, position)
        std::vector<int32_t> idx(static_cast<size_t>(nnz));
        for (int64_t k = 0; k < nnz; ++k) idx[k] = static_cast<int32_t>(k);
        auto less_mag = [&](int32_t a, int32_t b) {
            const float ma = std::fabs(vals[a]), mb = std::fabs(vals[b]);
            return ma < mb || (ma == mb && a < b);
        };
        if (n_prune > 0 && n_prune < nnz)
            std::nth_element(idx.begin(), idx.begin() + n_prune, idx.end(), less_mag);
        std::vector<char> pruned(static_cast<size_t>(nnz), 0);
        for (int64_t q = 0; q < n_prune; ++q) pruned[idx[q]] = 1;

        // 2. live set S as a bitmap over all O*I positions
        std::vector<uint64_t> live(static_cast<size_t>((cells + 63) / 64), 0);
        auto test_set = [&](uint64_t q) {
            uint64_t &w = live[q >> 6];
            const uint64_t bit = 1ULL << (q & 63);
            const bool was = (w & bit) != 0;
            w |= bit;
            return was;
        };
        for (int64_t k = 0; k < nnz; ++k)
            if (!pruned[k]) test_set(static_cast<uint64_t>(rows[k]) * I + cols[k]);

        // 3. regrow with Algorithm 2
        std::vector<uint64_t> grown;
        grown.reserve(static_cast<size_t>(n_prune));
        SplitMix64 rng{seed};
        int64_t trials = 0;
        while (static_cast<int64_t>(grown.size()) < n_prune) {
            const int64_t i = rng.below(O);
            const int64_t j = rng.below(I);
            ++trials;
            const uint64_t q = static_cast<uint64_t>(i) * I + j;
            if (test_set(q)) continue;
            grown.push_back(q);
        }
        std::sort(grown.begin(), grown.end());

        // 4. merge survivors (already sorted) with the sorted regrown positions
        int64_t at = 0;
        size_t g = 0;
        for (int64_t k = 0; k <= nnz; ++k) {
            const bool have_old = k < nnz;
            const uint64_t qold = have_old ? static_cast<uint64_t>(rows[k]) * I + cols[k] : ~0ULL;
            while (g < grown.size() && grown[g] < qold) {
                rows_out[at] = static_cast<int32_t>(grown[g] / I);
                cols_out[at] = static_cast<int32_t>(grown[g] % I);
                vals_out[at] = 0.0f;
                ++at;
                ++g;
            }
            if (have_old && !pruned[k]) {
                rows_out[at] = rows[k];
                cols_out[at] = cols[k];
                std::memcpy(&vals_out[at], &vals[k], sizeof(float));
                ++at;
            }
        }
        if (at != nnz) return fail(SNACK_ERR_INTERNAL, "topology: produced %lld entries", (long long)at);
        if (row_offsets_out) {
            std::fill(row_offsets_out, row_offsets_out + O + 1, 0);
            for (int64_t k = 0; k < nnz; ++k) ++row_offsets_out[rows_out[k] + 1];
            for (int64_t r = 0; r < O; ++r) row_offsets_out[r + 1] += row_offsets_out[r];
        }
        if (trials_out) *trials_out = trials;
        return ok();
    } catch (const std::bad_alloc &) {
        return fail(SNACK_ERR_NOMEM, "topology: out of host memory");
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "topology: unexpected exception");
    }
}
