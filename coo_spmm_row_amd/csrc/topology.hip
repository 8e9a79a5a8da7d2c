// topology.hip -- prune-and-regrow on the device (SNACK, Appendix G with the
// regrowth of Algorithm 2), giving the same triple, row offsets, column view and
// trial count as the host snack_coo_topology_update followed by the builder.
//
// 1. prune: the n_prune entries of smallest |vals|, ties by lower position: a sort
//    of the 64-bit keys (bits of |v|) << 32 | k.
// 2. the survivors, compacted in (row, col) order, and a bitmap of their cells
//    (each 32-bit word written by the one thread owning its first survivor).
// 3. regrowth: Algorithm 2 draws row = getrand(O) and col = getrand(I) from one
//    SplitMix64 stream and keeps a pair unless its cell is live (a survivor or an
//    earlier kept pair).  SplitMix64's i-th output depends only on seed + (i+1)*gamma,
//    so a batch of M draws is generated at once; sorting (cell, draw index) marks
//    each free cell's first draw, and in draw order the first `need` of those are
//    exactly the pairs the sequential loop keeps; the last one fixes the trial
//    count.  A batch that keeps fewer than `need` marks its cells live and the next
//    batch continues the stream.
// 4. survivors and regrown cells (value +0) merged by position (binary searches),
//    row offsets by binary search, and the column view by a sort on col*O + row.
#include <hip/hip_runtime.h>

#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "../../include/snack_coo.h"
#include "internal.h"

namespace snack {
namespace {

constexpr int kTB = 256;
constexpr int kDrawBits = 30;  // draw index within a batch in the low bits of the sort key
constexpr uint64_t kNoKey = ~0ULL;
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

inline unsigned blocks(int64_t n) { return static_cast<unsigned>((n + kTB - 1) / kTB); }

__device__ __forceinline__ uint64_t splitmix_output(uint64_t seed, uint64_t i) {  // i-th output, from 0
    uint64_t z = seed + (i + 1) * kGamma;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw_cell(uint64_t seed, uint64_t t, int64_t O, int64_t I) {
    const uint64_t r = __umul64hi(splitmix_output(seed, 2 * t), static_cast<uint64_t>(O));
    const uint64_t c = __umul64hi(splitmix_output(seed, 2 * t + 1), static_cast<uint64_t>(I));
    return r * static_cast<uint64_t>(I) + c;
}

template <typename T>
__device__ __forceinline__ int64_t lower_bound_dev(const T *a, int64_t n, T x) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a[mid] < x)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

template <typename T>
__global__ void fill_kernel(T *p, int64_t n, T v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void prune_keys_kernel(const float *vals, int64_t n, uint64_t *keys) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (k < n) keys[k] = (static_cast<uint64_t>(__float_as_uint(fabsf(vals[k]))) << 32) | static_cast<uint64_t>(k);
}

__global__ void mark_pruned_kernel(const uint64_t *sorted, int64_t p, int32_t *keep) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (i < p) keep[sorted[i] & 0xFFFFFFFFULL] = 0;
}

__global__ void survivors_kernel(const int32_t *rows, const int32_t *cols, const float *vals, const int32_t *keep,
                                 const int32_t *rank, int64_t n, int64_t I, uint64_t *spos, float *sval) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (k < n && keep[k]) {
        spos[rank[k]] = static_cast<uint64_t>(rows[k]) * static_cast<uint64_t>(I) + static_cast<uint64_t>(cols[k]);
        sval[rank[k]] = vals[k];
    }
}

// bitmap |= the cells of pos[0..n) (sorted, distinct): the thread holding the first cell of a
// 32-bit word ORs the word's whole run in, so every word has one writer
__global__ void bitmap_or_kernel(const uint64_t *pos, int64_t n, uint32_t *bitmap) {
    const int64_t s = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (s >= n) return;
    const uint64_t w = pos[s] >> 5;
    if (s > 0 && (pos[s - 1] >> 5) == w) return;
    uint32_t bits = 0;
    for (int64_t j = s; j < n && (pos[j] >> 5) == w; ++j) bits |= 1u << (pos[j] & 31);
    bitmap[w] |= bits;
}

__global__ void draw_kernel(uint64_t seed, uint64_t t0, int64_t m, int64_t O, int64_t I, const uint32_t *bitmap,
                            uint64_t *keys) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (t >= m) return;
    const uint64_t q = draw_cell(seed, t0 + static_cast<uint64_t>(t), O, I);
    const bool live = (bitmap[q >> 5] >> (q & 31)) & 1u;
    keys[t] = live ? kNoKey : ((q << kDrawBits) | static_cast<uint64_t>(t));
}

// fresh[t] = 1 for the first draw of each free cell (sorted keys: equal cells are adjacent,
// lowest draw index first)
__global__ void fresh_kernel(const uint64_t *sorted, int64_t m, int32_t *fresh) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (i >= m) return;
    const uint64_t key = sorted[i];
    if (key == kNoKey) return;
    const uint64_t q = key >> kDrawBits;
    if (i > 0 && (sorted[i - 1] >> kDrawBits) == q) return;
    fresh[key & ((1ULL << kDrawBits) - 1)] = 1;
}

// accepted draws (fresh, and among the first `need` fresh ones in draw order), flagged in
// cell order; the draw with rank need - 1 gives the trial count
__global__ void accept_kernel(const uint64_t *sorted, int64_t m, const int32_t *fresh, const int32_t *fscan,
                              int64_t need, int32_t *acc_sorted, int64_t *last_t) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (i >= m) return;
    const uint64_t key = sorted[i];
    int32_t a = 0;
    if (key != kNoKey) {
        const int64_t t = static_cast<int64_t>(key & ((1ULL << kDrawBits) - 1));
        if (fresh[t] && fscan[t] < need) {
            a = 1;
            if (fscan[t] == need - 1) *last_t = t;
        }
    }
    acc_sorted[i] = a;
}

__global__ void gather_accepted_kernel(const uint64_t *sorted, int64_t m, const int32_t *acc_sorted,
                                       const int32_t *acc_rank, uint64_t *out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (i < m && acc_sorted[i]) out[acc_rank[i]] = sorted[i] >> kDrawBits;
}

__global__ void merge_survivors_kernel(const uint64_t *spos, const float *sval, int64_t ns, const uint64_t *grown,
                                       int64_t ng, uint64_t *opos, float *oval) {
    const int64_t s = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (s >= ns) return;
    const int64_t j = s + lower_bound_dev(grown, ng, spos[s]);
    opos[j] = spos[s];
    oval[j] = sval[s];
}

__global__ void merge_grown_kernel(const uint64_t *grown, int64_t ng, const uint64_t *spos, int64_t ns, uint64_t *opos,
                                   float *oval) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (g >= ng) return;
    const int64_t j = g + lower_bound_dev(spos, ns, grown[g]);
    opos[j] = grown[g];
    oval[j] = 0.0f;
}

__global__ void emit_kernel(const uint64_t *opos, const float *oval, int64_t n, int64_t O, int64_t I, int32_t *rows,
                            int32_t *cols, float *vals, uint64_t *ckeys, uint32_t *cidx) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (j >= n) return;
    const uint64_t r = opos[j] / static_cast<uint64_t>(I), c = opos[j] % static_cast<uint64_t>(I);
    rows[j] = static_cast<int32_t>(r);
    cols[j] = static_cast<int32_t>(c);
    vals[j] = oval[j];
    ckeys[j] = c * static_cast<uint64_t>(O) + r;  // column view order: (col, row)
    cidx[j] = static_cast<uint32_t>(j);
}

// offsets[x] = number of sorted keys below x * stride, for x = 0..count
__global__ void offsets_kernel(const uint64_t *sorted, int64_t n, int64_t count, uint64_t stride, int32_t *offsets) {
    const int64_t x = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (x <= count) offsets[x] = static_cast<int32_t>(lower_bound_dev(sorted, n, static_cast<uint64_t>(x) * stride));
}

__global__ void colview_kernel(const uint64_t *ckeys, const uint32_t *cidx, int64_t n, int64_t O, int32_t *col_perm,
                               int32_t *col_rows, int32_t *col_cols) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kTB + threadIdx.x;
    if (j >= n) return;
    col_perm[j] = static_cast<int32_t>(cidx[j]);
    col_rows[j] = static_cast<int32_t>(ckeys[j] % static_cast<uint64_t>(O));
    col_cols[j] = static_cast<int32_t>(ckeys[j] / static_cast<uint64_t>(O));
}

int check_hip(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SNACK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return SNACK_OK;
}

int bits_for(uint64_t x) {  // bits needed to hold values < x
    int b = 1;
    while (b < 64 && (1ULL << b) < x) ++b;
    return b;
}

// H(n) = 1 + 1/2 + .. + 1/n (asymptotic series; exact enough for sizing a batch)
double harmonic(double n) {
    if (n < 1.0) return 0.0;
    if (n < 64.0) {
        double h = 0.0;
        for (int i = 1; i <= static_cast<int>(n); ++i) h += 1.0 / i;
        return h;
    }
    return std::log(n) + 0.5772156649015329 + 1.0 / (2.0 * n) - 1.0 / (12.0 * n * n);
}

// draws per batch: 1.25x the expected trial count (step i keeps a pair with probability
// (C - S - i) / C for C cells and S survivors) plus slack, within the key's index bits
int64_t draw_batch(int64_t O, int64_t I, int64_t nnz, int64_t n_prune) {
    if (const int64_t v = option(SNACK_OPT_TOPOLOGY_DRAW_BATCH); v > 0)
        return std::min<int64_t>(v, (int64_t(1) << kDrawBits) - 1);
    if (n_prune == 0) return 0;
    const double C = static_cast<double>(O) * static_cast<double>(I);
    const double free0 = C - static_cast<double>(nnz - n_prune);
    const double expect = C * (harmonic(free0) - harmonic(free0 - static_cast<double>(n_prune)));
    const double m = 1.25 * expect + 4096.0;
    return static_cast<int64_t>(std::min(m, static_cast<double>((int64_t(1) << kDrawBits) - 1)));
}

struct TopoPlan {
    int64_t m;  // draws per batch
    size_t off_ka, off_kb, off_keep, off_rank, off_spos, off_sval, off_bitmap, off_fresh, off_fscan, off_acc,
        off_accr, off_grown, off_opos, off_oval, off_cidx, off_cidx2, off_last, off_temp, temp_bytes, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int plan_topology(int64_t O, int64_t I, int64_t nnz, int64_t n_prune, TopoPlan &p) {
    p = TopoPlan{};
    p.m = draw_batch(O, I, nnz, n_prune);
    const int64_t nk = std::max<int64_t>(nnz, p.m) + 1;  // scans run over m + 1 flags
    const int64_t words = (O * I + 31) / 32;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        const size_t here = at;
        at = align256(at + std::max<size_t>(bytes, 1));
        return here;
    };
    p.off_ka = take(8 * nk);
    p.off_kb = take(8 * nk);
    p.off_keep = take(4 * (nnz + 1));
    p.off_rank = take(4 * (nnz + 1));
    p.off_spos = take(8 * (nnz + 1));
    p.off_sval = take(4 * (nnz + 1));
    p.off_bitmap = take(4 * static_cast<size_t>(words));
    p.off_fresh = take(4 * (p.m + 1));
    p.off_fscan = take(4 * (p.m + 1));
    p.off_acc = take(4 * (p.m + 1));
    p.off_accr = take(4 * (p.m + 1));
    p.off_grown = take(8 * (n_prune + 1));
    p.off_opos = take(8 * (nnz + 1));
    p.off_oval = take(4 * (nnz + 1));
    p.off_cidx = take(4 * (nnz + 1));
    p.off_cidx2 = take(4 * (nnz + 1));
    p.off_last = take(8);
    // temporary storage of the sorts and scans (sizes only: no device work)
    size_t t = 0, need = 0;
    hipcub::DoubleBuffer<uint64_t> kd(nullptr, nullptr);
    hipcub::DoubleBuffer<uint32_t> vd(nullptr, nullptr);
    if (hipcub::DeviceRadixSort::SortKeys(nullptr, t, kd, static_cast<int>(nk), 0, 64) != hipSuccess) return 1;
    need = std::max(need, t);
    if (hipcub::DeviceRadixSort::SortPairs(nullptr, t, kd, vd, static_cast<int>(std::max<int64_t>(nnz, 1)), 0, 64) !=
        hipSuccess)
        return 1;
    need = std::max(need, t);
    if (hipcub::DeviceScan::ExclusiveSum(nullptr, t, static_cast<int32_t *>(nullptr), static_cast<int32_t *>(nullptr),
                                         static_cast<int>(nk)) != hipSuccess)
        return 1;
    need = std::max(need, t);
    p.temp_bytes = need;
    p.off_temp = take(need);
    p.total = at;
    return 0;
}

}  // namespace
}  // namespace snack

using namespace snack;

extern "C" size_t snack_coo_topology_workspace_bytes(int64_t O, int64_t I, int64_t nnz, int64_t n_prune) {
    if (O <= 0 || I <= 0 || nnz < 0 || nnz > O * I || n_prune < 0 || n_prune > nnz || nnz > 2147483647LL ||
        static_cast<uint64_t>(O) * static_cast<uint64_t>(I) > (1ULL << 34)) {
        fail(SNACK_ERR_SHAPE, "topology_workspace_bytes: bad sizes");
        return 0;
    }
    TopoPlan p;
    if (plan_topology(O, I, nnz, n_prune, p)) {
        fail(SNACK_ERR_HIP, "topology_workspace_bytes: sort size query failed");
        return 0;
    }
    return p.total;
}

extern "C" int snack_coo_topology_update_device(const snack_coo_desc *W, int64_t n_prune, uint64_t seed,
                                                int32_t *rows_out, int32_t *cols_out, float *vals_out,
                                                int32_t *row_offsets_out, int32_t *col_perm_out,
                                                int32_t *col_rows_out, int32_t *col_cols_out,
                                                int32_t *col_offsets_out, int64_t *trials_out, void *workspace,
                                                size_t workspace_bytes, void *hip_stream) {
    try {
        const char *who = "topology_update_device";
        if (!W) return fail(SNACK_ERR_NULL, "%s: NULL descriptor", who);
        if (W->row_to_col)
            return fail(SNACK_ERR_UNSORTED, "%s: values in column order (row_to_col set); gather them into row "
                        "order first (snack_coo_gather_f32 with row_to_col)", who);
        const int64_t O = W->out_features, I = W->in_features, n = W->nnz;
        if (O <= 0 || I <= 0 || n < 0 || n > O * I || n_prune < 0 || n_prune > n || n > 2147483647LL)
            return fail(SNACK_ERR_SHAPE, "%s: bad sizes (O=%lld I=%lld nnz=%lld n_prune=%lld)", who, (long long)O,
                        (long long)I, (long long)n, (long long)n_prune);
        const uint64_t cells = static_cast<uint64_t>(O) * static_cast<uint64_t>(I);
        if (cells > (1ULL << 34)) return fail(SNACK_ERR_SHAPE, "%s: O*I exceeds the 2^34 bitmap limit", who);
        if (n > 0 && (!W->rows || !W->cols || !W->vals || !rows_out || !cols_out || !vals_out))
            return fail(SNACK_ERR_NULL, "%s: null array", who);
        if (!row_offsets_out || !col_offsets_out || (n > 0 && (!col_perm_out || !col_rows_out || !col_cols_out)))
            return fail(SNACK_ERR_NULL, "%s: null output", who);
        TopoPlan p;
        if (plan_topology(O, I, n, n_prune, p)) return fail(SNACK_ERR_HIP, "%s: sort size query failed", who);
        if (!workspace || workspace_bytes < p.total)
            return fail(SNACK_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, p.total,
                        workspace ? workspace_bytes : size_t(0));
        if (reinterpret_cast<uintptr_t>(workspace) % 256)
            return fail(SNACK_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        char *ws = static_cast<char *>(workspace);
        auto at = [&](size_t off) { return ws + off; };
        uint64_t *ka = reinterpret_cast<uint64_t *>(at(p.off_ka)), *kb = reinterpret_cast<uint64_t *>(at(p.off_kb));
        int32_t *keep = reinterpret_cast<int32_t *>(at(p.off_keep));
        int32_t *rank = reinterpret_cast<int32_t *>(at(p.off_rank));
        uint64_t *spos = reinterpret_cast<uint64_t *>(at(p.off_spos));
        float *sval = reinterpret_cast<float *>(at(p.off_sval));
        uint32_t *bitmap = reinterpret_cast<uint32_t *>(at(p.off_bitmap));
        int32_t *fresh = reinterpret_cast<int32_t *>(at(p.off_fresh));
        int32_t *fscan = reinterpret_cast<int32_t *>(at(p.off_fscan));
        int32_t *acc = reinterpret_cast<int32_t *>(at(p.off_acc));
        int32_t *accr = reinterpret_cast<int32_t *>(at(p.off_accr));
        uint64_t *grown = reinterpret_cast<uint64_t *>(at(p.off_grown));
        uint64_t *opos = reinterpret_cast<uint64_t *>(at(p.off_opos));
        float *oval = reinterpret_cast<float *>(at(p.off_oval));
        uint32_t *cidx = reinterpret_cast<uint32_t *>(at(p.off_cidx));
        uint32_t *cidx2 = reinterpret_cast<uint32_t *>(at(p.off_cidx2));
        int64_t *last_t = reinterpret_cast<int64_t *>(at(p.off_last));
        void *temp = at(p.off_temp);
        size_t temp_bytes = p.temp_bytes;  // reset before every call (the calls take it by reference)
        auto hip_ok = [&](hipError_t e, const char *what) {
            return e == hipSuccess ? SNACK_OK : fail(SNACK_ERR_HIP, "%s: %s: %s", who, what, hipGetErrorString(e));
        };
        const int64_t S = n - n_prune;

        // 1. prune set
        hipLaunchKernelGGL(fill_kernel<int32_t>, dim3(blocks(n + 1)), dim3(kTB), 0, st, keep, n + 1, 1);
        if (n_prune > 0) {
            hipLaunchKernelGGL(prune_keys_kernel, dim3(blocks(n)), dim3(kTB), 0, st, W->vals, n, ka);
            hipcub::DoubleBuffer<uint64_t> kd(ka, kb);
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceRadixSort::SortKeys(temp, temp_bytes, kd, static_cast<int>(n), 0, 63, st)),
                               "prune sort"))
                return s;
            hipLaunchKernelGGL(mark_pruned_kernel, dim3(blocks(n_prune)), dim3(kTB), 0, st, kd.Current(), n_prune, keep);
        }
        // 2. survivors and their bitmap
        if (n > 0) {
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceScan::ExclusiveSum(temp, temp_bytes, keep, rank, static_cast<int>(n), st)),
                               "survivor scan"))
                return s;
            hipLaunchKernelGGL(survivors_kernel, dim3(blocks(n)), dim3(kTB), 0, st, W->rows, W->cols, W->vals, keep, rank,
                               n, I, spos, sval);
        }
        const int64_t words = static_cast<int64_t>((cells + 31) / 32);
        hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3(blocks(words)), dim3(kTB), 0, st, bitmap, words, 0u);
        if (S > 0) hipLaunchKernelGGL(bitmap_or_kernel, dim3(blocks(S)), dim3(kTB), 0, st, spos, S, bitmap);
        if (int s = check_hip("topology_update_device setup")) return s;

        // 3. regrowth, one batch of draws at a time
        int64_t kept = 0, trials = 0;
        uint64_t t0 = 0;
        int batches = 0;
        while (kept < n_prune) {
            if (batches >= (1 << 16)) return fail(SNACK_ERR_INTERNAL, "%s: regrowth did not finish", who);
            const int64_t m = p.m, need = n_prune - kept;
            hipLaunchKernelGGL(draw_kernel, dim3(blocks(m)), dim3(kTB), 0, st, seed, t0, m, O, I, bitmap, ka);
            hipcub::DoubleBuffer<uint64_t> kd(ka, kb);
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceRadixSort::SortKeys(temp, temp_bytes, kd, static_cast<int>(m), 0, 64, st)),
                               "draw sort"))
                return s;
            const uint64_t *sorted = kd.Current();
            hipLaunchKernelGGL(fill_kernel<int32_t>, dim3(blocks(m + 1)), dim3(kTB), 0, st, fresh, m + 1, 0);
            hipLaunchKernelGGL(fresh_kernel, dim3(blocks(m)), dim3(kTB), 0, st, sorted, m, fresh);
            // exclusive scan over m + 1 flags (the last one 0): fscan[m] is the number of fresh draws
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceScan::ExclusiveSum(temp, temp_bytes, fresh, fscan, static_cast<int>(m + 1), st)),
                               "fresh scan"))
                return s;
            hipLaunchKernelGGL(fill_kernel<int64_t>, dim3(1), dim3(kTB), 0, st, last_t, int64_t(1), int64_t(-1));
            hipLaunchKernelGGL(accept_kernel, dim3(blocks(m)), dim3(kTB), 0, st, sorted, m, fresh, fscan, need, acc, last_t);
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceScan::ExclusiveSum(temp, temp_bytes, acc, accr, static_cast<int>(m), st)),
                               "accept scan"))
                return s;
            hipLaunchKernelGGL(gather_accepted_kernel, dim3(blocks(m)), dim3(kTB), 0, st, sorted, m, acc, accr,
                               grown + kept);
            int32_t nfresh = 0;
            int64_t last = -1;
            if (int s = hip_ok(hipMemcpyAsync(&nfresh, fscan + m, sizeof(int32_t), hipMemcpyDeviceToHost, st), "copy"))
                return s;
            if (int s = hip_ok(hipMemcpyAsync(&last, last_t, sizeof(int64_t), hipMemcpyDeviceToHost, st), "copy"))
                return s;
            if (int s = hip_ok(hipStreamSynchronize(st), "sync")) return s;
            if (nfresh >= need) {
                if (last < 0) return fail(SNACK_ERR_INTERNAL, "%s: no last accepted draw", who);
                trials = static_cast<int64_t>(t0) + last + 1;
                kept = n_prune;
            } else {
                // every fresh draw is kept: mark their cells live and continue the stream
                if (nfresh > 0)
                    hipLaunchKernelGGL(bitmap_or_kernel, dim3(blocks(nfresh)), dim3(kTB), 0, st, grown + kept,
                                       static_cast<int64_t>(nfresh), bitmap);
                kept += nfresh;
                t0 += static_cast<uint64_t>(m);
            }
            ++batches;
        }
        if (batches > 1) {  // each batch's cells are sorted; order them all
            hipcub::DoubleBuffer<uint64_t> kd(grown, ka);
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceRadixSort::SortKeys(temp, temp_bytes, kd, static_cast<int>(n_prune), 0,
                                                                 bits_for(cells), st)),
                               "regrown sort"))
                return s;
            if (kd.Current() != grown)
                if (int s = hip_ok(hipMemcpyAsync(grown, kd.Current(), 8 * n_prune, hipMemcpyDeviceToDevice, st), "copy"))
                    return s;
        }

        // 4. merged triple, row offsets, column view
        if (S > 0)
            hipLaunchKernelGGL(merge_survivors_kernel, dim3(blocks(S)), dim3(kTB), 0, st, spos, sval, S, grown, n_prune,
                               opos, oval);
        if (n_prune > 0)
            hipLaunchKernelGGL(merge_grown_kernel, dim3(blocks(n_prune)), dim3(kTB), 0, st, grown, n_prune, spos, S,
                               opos, oval);
        if (n > 0)
            hipLaunchKernelGGL(emit_kernel, dim3(blocks(n)), dim3(kTB), 0, st, opos, oval, n, O, I, rows_out, cols_out,
                               vals_out, ka, cidx);
        hipLaunchKernelGGL(offsets_kernel, dim3(blocks(O + 1)), dim3(kTB), 0, st, opos, n, O, static_cast<uint64_t>(I),
                           row_offsets_out);
        const uint64_t *ck = ka;
        if (n > 0) {
            hipcub::DoubleBuffer<uint64_t> kd(ka, kb);
            hipcub::DoubleBuffer<uint32_t> vd(cidx, cidx2);
            if (int s = hip_ok((temp_bytes = p.temp_bytes, hipcub::DeviceRadixSort::SortPairs(temp, temp_bytes, kd, vd, static_cast<int>(n), 0,
                                                                  bits_for(cells), st)),
                               "column sort"))
                return s;
            ck = kd.Current();
            hipLaunchKernelGGL(colview_kernel, dim3(blocks(n)), dim3(kTB), 0, st, ck, vd.Current(), n, O, col_perm_out,
                               col_rows_out, col_cols_out);
        }
        hipLaunchKernelGGL(offsets_kernel, dim3(blocks(I + 1)), dim3(kTB), 0, st, ck, n, I, static_cast<uint64_t>(O),
                           col_offsets_out);
        if (int s = check_hip("topology_update_device")) return s;
        if (trials_out) *trials_out = trials;
        return ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_topology_update_device: unexpected exception");
    }
}
