// snack_coo.hip -- device side of libsnack_coo for MI355X (gfx950, CDNA4, wave64).
//
// The SNACK layer (arXiv:2610.04093) keeps its weight W (O x I) as a COO triple
// sorted by (row, col) and runs three sparse products on it:
//   forward      Y[b,o]  = bias[o] + sum_{k: rows[k]=o} vals[k] X[b,cols[k]]   (Algorithm 1)
//   input grad   dX[b,i] = sum_{k: cols[k]=i} vals[k] dY[b,rows[k]]            (Section 3.4)
//   weight grad  dW[k]   = sum_b dY[b,rows[k]] X[b,cols[k]]                     (Section 3.4)
// The paper's CUDA mapping (Section 3.2: one thread per non-zero and batch
// column, atomics into C) is not used.  Here:
//  * activations are first laid out feature-major (A^T[f][b], fp32) so that the
//    operand row of one stored entry, A[:, f], is one contiguous vector;
//  * forward and input gradient are the same gather-reduce over a sorted
//    triple: the forward over the row order, the input gradient over the
//    column view (W^T with swapped indices, as Section 3.4 states), reading
//    vals through the column permutation.  Every output element is produced by
//    exactly one lane or by a fixed-order fix-up, so results are deterministic
//    and no atomics are used;
//  * two mappings of the gather-reduce:
//      segscan  - a wave owns a chunk of consecutive stored entries; lanes are
//                 (entry group g, batch lane t); row segments inside a step are
//                 combined by a segmented scan across entry groups; segments cut
//                 by a chunk edge go to a small partials buffer and are finished
//                 by fixup_kernel.  Balanced by nnz, so power-law rows are fine.
//      rowwave  - for batches that are multiples of 4: a wave owns one
//                 output row at a time; its entries are read 64 per coalesced
//                 load and prefetched a chunk ahead; lane slots gather float4s
//                 of the feature-major operand with several loads in flight.
//  * the weight gradient is a sampled dense-dense product over the stored
//    entries: a group of BT lanes per entry, each lane a slice of the batch,
//    reduced across the group by xor shuffles.
//  * LDS-tiled forms of all three (large layers, batches padded to a multiple
//    of 16 up to 256): W is cut into tiles of a key range x a block of ~625
//    operand rows; a 1024-thread workgroup stages its block of the operand in
//    LDS once and serves every entry of the tile from there (tile_spmm_kernel,
//    tile_sddmm_kernel, tile_bwd_kernel); the forward and input gradient write
//    per-block partial sums that tile_sum_kernel adds in block order.
// No MFMA: the work is an irregular gather, not a dense contraction.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/snack_coo.h"
#include "internal.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;               // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kXcds = 8;                  // MI355X: 8 accelerator dies, round-robin dispatch
constexpr int64_t kMaxBatch = int64_t(1) << 21;  // keeps every grid.y within 65535

typedef uint16_t bf16_t;

// ---------------------------------------------------------------- element I/O
__device__ __forceinline__ float load_act(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_act(const bf16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ __forceinline__ void store_act(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_act(bf16_t *p, int64_t i, float v) {
    // round to nearest, ties to even; NaN stays a quiet NaN
    uint32_t u = __float_as_uint(v);
    uint16_t h;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
        h = static_cast<uint16_t>((u >> 16) | 0x0040u);
    } else {
        h = static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    p[i] = h;
}

// Cross-lane moves within a row of 16 lanes (DPP).  Controls: quad_perm
// [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16); every lane of the
// group receives the group's sum.  The pairings (xor 1, xor 2, mirror within 8,
// mirror within 16) form a butterfly, so each step adds two disjoint partial sums.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_move<0xB1>(v);
    if constexpr (N >= 4) v += dpp_move<0x4E>(v);
    if constexpr (N >= 8) v += dpp_move<0x141>(v);
    if constexpr (N >= 16) v += dpp_move<0x140>(v);
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
    return v;
}

// Reduce-scatter of U values over aligned groups of N lanes (U <= N, both powers of two):
// lane t of a group returns the group's sum of v[t / (N / U)].  The stages pair lanes by
// mirror within 16 (xor 15), mirror within 8 (xor 7), xor 2 and xor 1 -- the last log2(N) of
// these, an independent set of lane masks, so every stage adds disjoint partial sums.  While
// more than one value is left, a lane keeps the half its own bit selects (bit 3, 2, 1, 0 of
// the lane in those stages), and sends the other half to its partner, which differs in that
// bit; once one value is left the remaining stages are plain reductions.  That is log2(U)
// halvings (3 instructions per kept value) plus one add per further stage, against U full
// group sums of log2(N) adds each.
// One stage of group_reduce_scatter: M values live in w[0, M); partner = the DPP source lane.
template <int CTRL, int BIT, int M, int U>
__device__ __forceinline__ void reduce_scatter_stage(float (&w)[U], int t) {
    if constexpr (M > 1) {
        constexpr int H = M / 2;
        const bool hi = (t >> BIT) & 1;
#pragma unroll
        for (int j = 0; j < H; ++j) {
            const float send = hi ? w[j] : w[j + H];
            const float keep = hi ? w[j + H] : w[j];
            w[j] = keep + dpp_move<CTRL>(send);
        }
    } else {
        w[0] += dpp_move<CTRL>(w[0]);
    }
}

template <int N, int U>
__device__ __forceinline__ float group_reduce_scatter(const float (&v)[U], int t) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
    static_assert(U >= 1 && U <= N && (U & (U - 1)) == 0, "U a power of two <= N");
    float w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) w[j] = v[j];
    constexpr int M0 = U;
    if constexpr (N >= 16) reduce_scatter_stage<0x140, 3, M0, U>(w, t);
    constexpr int M1 = N >= 16 && M0 > 1 ? M0 / 2 : M0;
    if constexpr (N >= 8) reduce_scatter_stage<0x141, 2, M1, U>(w, t);
    constexpr int M2 = N >= 8 && M1 > 1 ? M1 / 2 : M1;
    if constexpr (N >= 4) reduce_scatter_stage<0x4E, 1, M2, U>(w, t);
    constexpr int M3 = N >= 4 && M2 > 1 ? M2 / 2 : M2;
    if constexpr (N >= 2) reduce_scatter_stage<0xB1, 0, M3, U>(w, t);
    return w[0];
}

// Logical workgroup index such that each XCD (blockIdx.x % 8 under round-robin
// dispatch) works on one contiguous eighth of the logical range.  gridDim.x is
// a multiple of 8; callers drop logical ids beyond their real count.
__device__ __forceinline__ int64_t xcd_block() {
    const int64_t per = gridDim.x / kXcds;
    return (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

// ---------------------------------------------------------------- layout
// in [B][F] (batch-major, fp32 or bf16)  ->  out [F+1][Bp] fp32 (feature-major, Bp >= B; columns
// B..Bp-1 zero), row F zero (gathers of a missing entry point there instead of being masked).
// Up to two tensors per launch (blockIdx.z; the backward pass transposes X and dY together).
// A workgroup moves a tile of 32 features x 64 batch rows through LDS.
constexpr int kTf = 32, kTb = 64;

// Any F and B: each thread issues its eight scalar loads (128-byte row segments per 32 lanes)
// before its stores; the tile's output is one contiguous run per feature.
template <typename InT>
__global__ __launch_bounds__(kBlock) void to_feature_major_kernel(const InT *__restrict__ in0,
                                                                  float *__restrict__ out0, int64_t F0,
                                                                  const InT *__restrict__ in1,
                                                                  float *__restrict__ out1, int64_t F1,
                                                                  int64_t B, int64_t Bp) {
    __shared__ float tile[kTb][kTf + 1];
    const InT *__restrict__ in = blockIdx.z == 0 ? in0 : in1;
    float *__restrict__ out = blockIdx.z == 0 ? out0 : out1;
    const int64_t F = blockIdx.z == 0 ? F0 : F1;
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTf;
    if (f0 >= F && !(blockIdx.x == 0)) return;  // uniform per workgroup, before the barrier
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTb;
    const int tx = threadIdx.x % kTf, ty = threadIdx.x / kTf;  // 32 x 8
    const int nb = static_cast<int>(max<int64_t>(0, min<int64_t>(kTb, B - b0)));
    const int nbp = static_cast<int>(min<int64_t>(kTb, Bp - b0));  // with the zero columns
    const int nf = static_cast<int>(max<int64_t>(0, min<int64_t>(kTf, F - f0)));
    if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < nbp) out[F * Bp + b0 + threadIdx.x] = 0.f;
    constexpr int K = kTb / (kBlock / kTf);  // 8 rows per thread
    float v[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int bb = ty + (kBlock / kTf) * i;
        v[i] = (bb < nb && tx < nf) ? load_act(in, (b0 + bb) * F + f0 + tx) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) tile[ty + (kBlock / kTf) * i][tx] = v[i];
    __syncthreads();
    for (int li = threadIdx.x; li < nf * nbp; li += kBlock) {  // rows nb..nbp-1 of the tile are zero
        const int ff = li / nbp, bb = li % nbp;
        out[(f0 + ff) * Bp + b0 + bb] = tile[bb][ff];
    }
}

__device__ __forceinline__ float4 load_act4(const float *p, int64_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
}
__device__ __forceinline__ float4 load_act4(const bf16_t *p, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xFFFF0000u));
}

// F and Bp multiples of 4 (16-byte aligned rows): each thread loads two 4-feature vectors of
// two batch rows (zeros past B) and stores two 4-row vectors of two features, with no divisions.  LDS rows
// are padded to 33 floats: the 4 scalar writes and reads of a vector fall in distinct banks.
template <typename InT>
__global__ __launch_bounds__(kBlock) void to_feature_major4_kernel(const InT *__restrict__ in0,
                                                                   float *__restrict__ out0, int64_t F0,
                                                                   const InT *__restrict__ in1,
                                                                   float *__restrict__ out1, int64_t F1,
                                                                   int64_t B, int64_t Bp) {
    __shared__ float tile[kTb][kTf + 1];
    const InT *__restrict__ in = blockIdx.z == 0 ? in0 : in1;
    float *__restrict__ out = blockIdx.z == 0 ? out0 : out1;
    const int64_t F = blockIdx.z == 0 ? F0 : F1;
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTf;
    if (f0 >= F && !(blockIdx.x == 0)) return;  // uniform per workgroup, before the barrier
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTb;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && b0 + tid < Bp && tid < kTb) out[F * Bp + b0 + tid] = 0.f;
    // load: thread -> batch row r = tid / 8 (+32), features 4 * (tid % 8) .. +3
    const int lc = 4 * (tid % (kTf / 4)), lr = tid / (kTf / 4);
    float4 v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t b = b0 + lr + 32 * i, f = f0 + lc;
        v[i] = (b < B && f < F) ? load_act4(in, b * F + f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float *t = &tile[lr + 32 * i][lc];
        t[0] = v[i].x;
        t[1] = v[i].y;
        t[2] = v[i].z;
        t[3] = v[i].w;
    }
    __syncthreads();
    // store: thread -> feature ff = tid / 16 (+16), batch rows 4 * (tid % 16) .. +3
    const int sq = 4 * (tid % (kTb / 4)), sf = tid / (kTb / 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ff = sf + 16 * i;
        const int64_t f = f0 + ff, b = b0 + sq;
        if (f < F && b < Bp)
            *reinterpret_cast<float4 *>(out + f * Bp + b) =
                make_float4(tile[sq][ff], tile[sq + 1][ff], tile[sq + 2][ff], tile[sq + 3][ff]);
    }
}

// ---------------------------------------------------------------- segscan mapping
// keys[k]  : output index of entry k (row for the forward, column for dX), sorted
// gidx[k]  : operand row gathered by entry k (column for the forward, row for dX)
// vals[perm ? perm[k] : k] : the entry's value
// opnd     : feature-major operand [*][B]
// out[b * out_ld + key] = bias[key] + sum over the key's entries
// head/tail[chunk][B]   : partial sums of segments cut by a chunk edge
template <int BT, typename OutT>
__global__ __launch_bounds__(kBlock) void segscan_kernel(
    int64_t nnz, int64_t chunk, int64_t nchunks, const int32_t *__restrict__ keys,
    const int32_t *__restrict__ gidx, const float *__restrict__ vals, const int32_t *__restrict__ perm,
    const float *__restrict__ opnd, int64_t B, const float *__restrict__ bias, OutT *__restrict__ out,
    int64_t out_ld, float *__restrict__ head, float *__restrict__ tail) {
    constexpr int G = kWave / BT;
    constexpr int U = 4;  // steps whose loads are issued together
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT, t = lane % BT;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
    if (j >= nchunks) return;  // uniform per wave
    const int64_t b = static_cast<int64_t>(blockIdx.y) * BT + t;
    const bool bok = b < B;
    const int64_t kbeg = j * chunk;
    const int64_t kend = min(kbeg + chunk, nnz);
    const int prev_key = kbeg > 0 ? keys[kbeg - 1] : -1;
    const int next_key = kend < nnz ? keys[kend] : -1;
    const int first_key = keys[kbeg];
    float carry = 0.f;
    int carry_key = -4;
    for (int64_t base = kbeg; base < kend; base += U * G) {
        int key[U], nkey[U];
        float p[U];
        int64_t c[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + u * G + g;
            key[u] = -2;
            nkey[u] = -3;
            c[u] = 0;
            v[u] = 0.f;
            if (k < kend) {
                key[u] = keys[k];
                nkey[u] = (k + 1 < kend) ? keys[k + 1] : -3;
                v[u] = vals[perm ? static_cast<int64_t>(perm[k]) : k];
                c[u] = gidx[k];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) p[u] = (key[u] != -2 && bok) ? v[u] * opnd[c[u] * B + b] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = base + u * G + g;
            // segmented inclusive scan across the G entry groups (keys are sorted,
            // so equal keys at distance d mean the whole span shares the key)
#pragma unroll
            for (int d = 1; d < G; d <<= 1) {
                const float up = __shfl_up(p[u], d * BT, kWave);
                const int upkey = __shfl_up(key[u], d * BT, kWave);
                if (g >= d && upkey == key[u]) p[u] += up;
            }
            if (key[u] == carry_key) p[u] += carry;
            carry = __shfl(p[u], (G - 1) * BT + t, kWave);
            carry_key = __shfl(key[u], (G - 1) * BT + t, kWave);
            if (key[u] != -2 && bok && nkey[u] != key[u]) {
                const bool cut_left = key[u] == prev_key;
                const bool cut_right = (k == kend - 1) && key[u] == next_key;
                if (cut_left || cut_right) {
                    if (key[u] == first_key)
                        head[j * B + b] = p[u];
                    else
                        tail[j * B + b] = p[u];
                } else {
                    store_act(out, b * out_ld + key[u], p[u] + (bias ? bias[key[u]] : 0.f));
                }
            }
        }
    }
}

// Finishes keys with no entries (output = bias) and keys whose entries span
// several chunks (sum of the chunk partials in chunk order, then the bias).
template <typename OutT>
__global__ __launch_bounds__(kBlock) void fixup_kernel(int64_t nkeys, int64_t B, int64_t chunk,
                                                       const int32_t *__restrict__ offs,
                                                       const float *__restrict__ bias,
                                                       const float *__restrict__ head,
                                                       const float *__restrict__ tail,
                                                       OutT *__restrict__ out, int64_t out_ld) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (r >= nkeys) return;
    const float bv = bias ? bias[r] : 0.f;
    const int64_t s = offs[r], e = offs[r + 1];
    for (int64_t b = blockIdx.y; b < B; b += gridDim.y) {
        if (s == e) {
            store_act(out, b * out_ld + r, bv);
            continue;
        }
        const int64_t cs = s / chunk, ce = (e - 1) / chunk;
        if (cs == ce) continue;  // written by segscan_kernel
        float v = (s == cs * chunk) ? head[cs * B + b] : tail[cs * B + b];
        for (int64_t c = cs + 1; c <= ce; ++c) v += head[c * B + b];
        store_act(out, b * out_ld + r, v + bv);
    }
}

// ---------------------------------------------------------------- rowwave mapping
// For batches that are multiples of 4.  A workgroup of 4 waves owns 4/WPR
// output keys (rows), each split over WPR waves.  Lanes are (slot e, lane t):
// S = 64/BT slots each take one stored entry per step, lane t holds batch
// columns b0+4t .. b0+4t+3 and, with Q > 1, the float4s t+BT, .., t+(Q-1)BT
// further on (the batch tile is 4*BT*Q columns; Q > 1 only when tiles are
// exact).  A wave reads its key's entries 64 at a time (chunks c, c+WPR, ...)
// with one coalesced load per lane -- keeping each entry's operand row as a
// 32-bit float4 offset -- prefetches its next chunk while the current one is
// consumed, and keeps U*Q float4 gathers in flight.  Lanes of a chunk past the
// key's end point at the operand's zero row with value 0, so no step needs a
// mask.  Slot partial sums are combined by xor shuffles, the WPR waves of a
// key through LDS.  The operand including its zero row is below 4 GB.  B is the operand's batch
// columns (a multiple of 4; zero columns pad a batch of nbo columns), nbo the columns stored.
template <int BT, int WPR, int Q, typename OutT>
__global__ __launch_bounds__(kBlock) void rowwave_kernel(
    int64_t nkeys, const int32_t *__restrict__ offs, const int32_t *__restrict__ gidx,
    const float *__restrict__ vals, const int32_t *__restrict__ perm, const float *__restrict__ opnd, int zero_row,
    int64_t B, const float *__restrict__ bias, OutT *__restrict__ out, int64_t out_ld, int64_t nbo) {
    constexpr int S = kWave / BT;
    constexpr int UQ = 8 / Q;
    constexpr int U = (S * UQ <= kWave) ? UQ : kWave / S;  // S*U divides 64
    constexpr int KPB = kWavesPerBlock / WPR;             // keys per workgroup
    __shared__ float4 part[kWavesPerBlock][Q][BT];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int e = lane / BT, t = lane % BT;
    const int64_t r = xcd_block() * KPB + wave / WPR;
    const int wsub = wave % WPR;
    const bool rok = r < nkeys;  // uniform per wave
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * (4 * BT * Q) + 4 * t;
    const bool bok = b0 < B;     // B % 4 == 0: all four columns exist (Q > 1: every lane)
    const int B4 = static_cast<int>(B / 4);
    // uniform base of this batch tile; a lane adds its float4 column and the entry's row
    const char *__restrict__ tile = reinterpret_cast<const char *>(opnd) + blockIdx.y * (16 * BT * Q);
    const uint32_t lane_off = 16u * static_cast<uint32_t>(bok ? t : 0);
    float4 acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (rok) {
        const int zoff = zero_row * B4;
        const int s = offs[r], end = offs[r + 1];
        int mo = zoff;
        float mv = 0.f;
        const int first = s + wsub * kWave;
        if (first + lane < end) {
            mo = gidx[first + lane] * B4;
            mv = vals[perm ? perm[first + lane] : first + lane];
        }
        for (int base = first; base < end; base += WPR * kWave) {
            const int co = mo;
            const float cv = mv;
            const int n = min(kWave, end - base);
            const int nb = base + WPR * kWave;
            if (nb < end) {  // prefetch this wave's next chunk
                mo = zoff;
                mv = 0.f;
                if (nb + lane < end) {
                    mo = gidx[nb + lane] * B4;
                    mv = vals[perm ? perm[nb + lane] : nb + lane];
                }
            }
            for (int h = 0; h < n; h += S * U) {
                const int sa = (h + e) << 2;  // ds_bpermute address of slot e's entry; +4S per step
                float4 x[U][Q];
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int o = __builtin_amdgcn_ds_bpermute(sa + 4 * S * u, co);
                    v[u] = __int_as_float(__builtin_amdgcn_ds_bpermute(sa + 4 * S * u, __float_as_int(cv)));
                    const uint32_t a = 16u * static_cast<uint32_t>(o) + lane_off;
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        x[u][q] = *reinterpret_cast<const float4 *>(tile + (a + 16u * static_cast<uint32_t>(q * BT)));
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        acc[q].x = fmaf(v[u], x[u][q].x, acc[q].x);
                        acc[q].y = fmaf(v[u], x[u][q].y, acc[q].y);
                        acc[q].z = fmaf(v[u], x[u][q].z, acc[q].z);
                        acc[q].w = fmaf(v[u], x[u][q].w, acc[q].w);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
        for (int d = BT; d < kWave; d <<= 1) {
            acc[q].x += __shfl_xor(acc[q].x, d, kWave);
            acc[q].y += __shfl_xor(acc[q].y, d, kWave);
            acc[q].z += __shfl_xor(acc[q].z, d, kWave);
            acc[q].w += __shfl_xor(acc[q].w, d, kWave);
        }
    }
    if constexpr (WPR > 1) {
        if (e == 0) {
#pragma unroll
            for (int q = 0; q < Q; ++q) part[wave][q][t] = acc[q];
        }
        __syncthreads();
        if (wsub == 0 && e == 0) {
#pragma unroll
            for (int w = 1; w < WPR; ++w) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 o = part[wave + w][q][t];
                    acc[q].x += o.x;
                    acc[q].y += o.y;
                    acc[q].z += o.z;
                    acc[q].w += o.w;
                }
            }
        }
    }
    if (rok && wsub == 0 && e == 0 && bok) {
        const float bv = bias ? bias[r] : 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t c = b0 + 4 * q * BT;
            if (c + 3 < nbo) {
                store_act(out, (c + 0) * out_ld + r, acc[q].x + bv);
                store_act(out, (c + 1) * out_ld + r, acc[q].y + bv);
                store_act(out, (c + 2) * out_ld + r, acc[q].z + bv);
                store_act(out, (c + 3) * out_ld + r, acc[q].w + bv);
            } else {  // the last, padded float4 of the batch
                if (c + 0 < nbo) store_act(out, (c + 0) * out_ld + r, acc[q].x + bv);
                if (c + 1 < nbo) store_act(out, (c + 1) * out_ld + r, acc[q].y + bv);
                if (c + 2 < nbo) store_act(out, (c + 2) * out_ld + r, acc[q].z + bv);
            }
        }
    }
}

// ---------------------------------------------------------------- LDS-tiled gather-reduce
// The same gather-reduce as rowwave (out[key][:] = sum over the key's entries of
// vals * opnd[gidx][:]), with the operand rows served from LDS instead of L2.  W is cut into
// tiles of (a range of keys) x (a block of cw operand rows); a 1024-thread workgroup stages its
// block of the feature-major operand (cw rows of 64 batch columns, 256 B each, plus one zero
// row: up to 160 KB, gfx950's LDS) once, then walks its keys' segments inside the block.  The
// segments come from a per-block segment list (tile_segments_kernel; the triple is sorted by key,
// then by gather index, so each segment is a contiguous run of the key's entries), whose keys are
// ordered by segment length within windows of kSegWindow keys: the four keys a wave walks together
// have segments of about the same length, so little of the walk is padding.  Each tile writes fp32
// partial sums part[bt][cb][key][64]; tile_sum_kernel adds the blocks in block order, adds the
// bias and transposes to the batch-major output.
//
// Lanes: 4 slots of 16 lanes; slot s walks key 4*g + s of the wave's group g, and each lane holds
// VW batch columns (VW floats) of a TB = 16*VW column batch tile (64 for batches padded to a
// multiple of 64, else 32 or 16).  A group's entries are loaded 16 per chunk register (each row
// of 16 lanes holds entries j = 0..15 of its slot's chunk), two groups ahead of the compute.
// Step t of a chunk hands entry t to every lane of its row with DPP row_newbcast:t: folded into
// the row address (an XOR), and moved once into a register for the value, so one step costs one
// LDS read of VW floats per lane, an address XOR, a value move and VW plain FMAs.  Entries past a
// segment's end point at the zero row with value 0.
constexpr int kTileThreads = 1024;
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kTileLdsRows = 639;                     // staged rows: 159.75 KB of LDS at 64 columns
constexpr int kTileMaxCols = kTileLdsRows - 1;        // operand rows per block (one more is the zero row)
constexpr int kTileClaimBytes = 16;                   // after the staged rows: the workgroup's group counter

// Raw buffer resource over n 4-byte elements: loads through it take a 32-bit byte offset (the
// chunk offsets fold into the instruction's immediate), and loads past the end return 0 instead of
// touching memory.  Word 3 is the gfx9 raw-buffer format.  Callers keep n < 2^29, so byte offsets
// of elements stay below 2^31 and below kBufPast.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), n * 4, 0x00020000);
}
__device__ __forceinline__ int buf_ld(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
constexpr int kBufPast = static_cast<int>(0xFFFFFFF0u);  // a byte offset past any buffer: the load returns 0

// lane T of each row of 16 lanes, broadcast to the row (DPP row_newbcast)
template <int T>
__device__ __forceinline__ uint32_t bcast16(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x150 + T, 0xF, 0xF, true));
}

template <int SL>
struct TileVec;
template <>
struct TileVec<1> { typedef float T; };
template <>
struct TileVec<2> { typedef float2 T; };
template <>
struct TileVec<4> { typedef float4 T; };

__device__ __forceinline__ float vget(const float &v, int) { return v; }
__device__ __forceinline__ float vget(const float2 &v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ float vget(const float4 &v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Staged rows of the tiled walks that read the activations in place (tile_spmm_kernel,
// tile_sddmm_kernel): row r holds TB = 16 VW fp32 batch columns as NQ = TB / 4 chunks of 16 bytes,
// chunk q (columns 4q .. 4q+3) at chunk position q ^ (r & kSwz).  Staging writes one chunk per
// thread for consecutive rows; unswizzled, those writes would all hit the same four banks.  On
// gfx950 a 128-bit LDS read by four slots of 16 lanes, each slot reading one row, runs at the full
// rate only while the slots' chunk positions differ in their two low bits at most (measured: XOR of
// the low two bits 232 B/clk/CU; XOR of all four bits by row 169; the writes reach 62 of at most
// 72 B/clk/CU with the low two bits), hence kSwz = 3.  Lane byte offsets below 16 NQ and row
// offsets that are multiples of 16 NQ combine as row_off(r) ^ lane_off, row_off(r) = r * 16 NQ +
// 16 (r & kSwz): the XOR replaces the address add of an unswizzled row.
constexpr int kSwz = 3;

template <int VW>
__device__ __forceinline__ uint32_t tile_row_off(int r) {
    constexpr int NQ = 4 * VW;
    return static_cast<uint32_t>(r) * (16u * NQ) + 16u * static_cast<uint32_t>(r & kSwz);
}

// Buffer resource over an activation of n elements (fp32 or bf16) and a load of one element,
// widened to fp32: past the end, or at kBufPast, the load returns 0.  Callers keep n * the element
// size below 2^31.
template <typename InT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const InT *p, int n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<InT *>(p), static_cast<short>(0),
                                             n * static_cast<int>(sizeof(InT)), 0x00020000);
}
template <typename InT>
__device__ __forceinline__ float act_ld(__amdgpu_buffer_rsrc_t r, int byte_off);
template <>
__device__ __forceinline__ float act_ld<float>(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
template <>
__device__ __forceinline__ float act_ld<bf16_t>(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0)) << 16);
}

// Stages rows [r0, r0 + cn) (feature index) of batch tile bt of a batch-major activation [B][ld]
// (fp32 or bf16, widened to fp32; ra = act_rsrc over its B * ld elements) into LDS rows 0 .. cn-1
// in the swizzled layout above; rows cn .. cw (row cw is the zero row) and batch rows >= B are
// zero (loaded past the buffer).  Item i is chunk q = i / 640 of row c = i % 640 (640 =
// kTileLdsRows + 1 >= cw + 1, a constant divisor): consecutive threads take consecutive rows of
// one chunk, so each of a chunk's four batch rows is read in runs of 64 features.
template <int VW, typename InT>
__device__ __forceinline__ void tile_stage_rows(float4 *xs4, __amdgpu_buffer_rsrc_t ra, int ld, int bt, int r0,
                                                int cn, int cw) {
    constexpr int NQ = 4 * VW, TB = 16 * VW, kStride = kTileLdsRows + 1;
    constexpr int kEs = static_cast<int>(sizeof(InT));
    constexpr int kIters = (kStride * NQ + kTileThreads - 1) / kTileThreads;
    constexpr int kRound = kIters < 5 ? kIters : 5;  // items whose loads are in flight together
#pragma unroll
    for (int it0 = 0; it0 < kIters; it0 += kRound) {
        float4 v[kRound];
        int at[kRound];
#pragma unroll
        for (int u = 0; u < kRound && it0 + u < kIters; ++u) {
            const int i = (it0 + u) * kTileThreads + static_cast<int>(threadIdx.x);
            const int q = i / kStride, c = i - q * kStride;
            at[u] = q < NQ && c <= cw ? c * NQ + (q ^ (c & kSwz)) : -1;
            const int off = q < NQ && c < cn ? ((TB * bt + 4 * q) * ld + r0 + c) * kEs : kBufPast;
            const int step = off == kBufPast ? 0 : ld * kEs;
            v[u] = make_float4(act_ld<InT>(ra, off), act_ld<InT>(ra, off + step), act_ld<InT>(ra, off + 2 * step),
                               act_ld<InT>(ra, off + 3 * step));
        }
#pragma unroll
        for (int u = 0; u < kRound && it0 + u < kIters; ++u)
            if (at[u] >= 0) xs4[at[u]] = v[u];
    }
}

// The LDS reads of steps T0..T0+3 of one chunk (entry T0+u's staged row, this lane's VW columns;
// off is the entry's tile_row_off).
template <int VW, int T0>
__device__ __forceinline__ void tile_reads4(typename TileVec<VW>::T (&x)[4], uint32_t off, uint32_t lane_off,
                                            const char *lds) {
    typedef typename TileVec<VW>::T V;
    x[0] = *reinterpret_cast<const V *>(lds + (bcast16<T0 + 0>(off) ^ lane_off));
    x[1] = *reinterpret_cast<const V *>(lds + (bcast16<T0 + 1>(off) ^ lane_off));
    x[2] = *reinterpret_cast<const V *>(lds + (bcast16<T0 + 2>(off) ^ lane_off));
    x[3] = *reinterpret_cast<const V *>(lds + (bcast16<T0 + 3>(off) ^ lane_off));
}

// Lane T of each row of 16 lanes' v, broadcast to the row, in a register of its own (inline asm,
// so the compiler does not fold the DPP move into the FMAs that use it: a DPP FMA issues at about
// 0.77 per clock per CU, a plain one at the full rate).  NOP1: the two wait states a VALU write of
// v needs before a DPP read, on the first step of a chunk; volatile keeps the moves of a chunk in
// step order, so that one runs first (the compiler adds no wait states for inline asm).
template <int T, bool NOP1>
__device__ __forceinline__ float bcast16_reg(float v) {
    float r;
    if constexpr (NOP1)
        asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                     : "=v"(r) : "v"(v), "n"(T));
    else
        asm volatile("v_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                     : "=v"(r) : "v"(v), "n"(T));
    return r;
}

// The FMAs of steps T0..T0+3: acc += (value of entry T0+u) * row.
template <int VW, int T0>
__device__ __forceinline__ void tile_fmas4(float (&acc)[VW], float v, const typename TileVec<VW>::T (&x)[4]) {
    const float v0 = bcast16_reg<T0 + 0, T0 == 0>(v), v1 = bcast16_reg<T0 + 1, false>(v);
    const float v2 = bcast16_reg<T0 + 2, false>(v), v3 = bcast16_reg<T0 + 3, false>(v);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
        acc[i] = fmaf(v0, vget(x[0], i), acc[i]);
        acc[i] = fmaf(v1, vget(x[1], i), acc[i]);
        acc[i] = fmaf(v2, vget(x[2], i), acc[i]);
        acc[i] = fmaf(v3, vget(x[3], i), acc[i]);
    }
}

// One chunk of 16 entries, nst (uniform, 1..16) of them real for the longest slot.  The reads of
// each group of four steps are issued before the FMAs of the group before it, so a wave has a
// group's LDS reads in flight while it computes.
template <int VW>
__device__ __forceinline__ void tile_chunk(float (&acc)[VW], uint32_t off, float v, int nst, uint32_t lane_off,
                                           const char *lds) {
    typedef typename TileVec<VW>::T V;
    V a[4], b[4];
    tile_reads4<VW, 0>(a, off, lane_off, lds);
    if (nst > 4) tile_reads4<VW, 4>(b, off, lane_off, lds);
    tile_fmas4<VW, 0>(acc, v, a);
    if (nst > 4) {
        if (nst > 8) tile_reads4<VW, 8>(a, off, lane_off, lds);
        tile_fmas4<VW, 4>(acc, v, b);
        if (nst > 8) {
            if (nst > 12) tile_reads4<VW, 12>(b, off, lane_off, lds);
            tile_fmas4<VW, 8>(acc, v, a);
            if (nst > 12) tile_fmas4<VW, 12>(acc, v, b);
        }
    }
}

// Segment lists: seg[j][p] (int32 x 4) = {key, start, end, 0} for block j (gather indices
// [j cw, j cw + cw)) and list position p: the key's entries in the block are [start, end).  Within
// each window of kSegWindow positions [w kSegWindow, w kSegWindow + kSegWindow) the keys are those
// of the same window, by decreasing end - start, equal lengths by increasing key.  One wave per
// (block, window): lane l finds key w kSegWindow + l's segment by binary search and its rank by
// comparing with every other lane's length.
constexpr int kSegWindow = 32;  // 32 consecutive keys: one 128-byte line of a batch-major row

__device__ __forceinline__ int first_at_or_past(const int32_t *__restrict__ gidx, int lo, int hi, int c) {
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (gidx[mid] < c) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(kBlock) void tile_segments_kernel(int nkeys, int ncb, int cw,
                                                               const int32_t *__restrict__ offs,
                                                               const int32_t *__restrict__ gidx,
                                                               int4 *__restrict__ seg) {
    const int nwin = (nkeys + kSegWindow - 1) / kSegWindow;
    const int64_t wv = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) / kWave;  // uniform per wave
    if (wv >= static_cast<int64_t>(ncb) * nwin) return;
    const int j = static_cast<int>(wv / nwin), w = static_cast<int>(wv % nwin);
    const int lane = threadIdx.x & (kWave - 1);
    const int key = w * kSegWindow + lane;
    const bool real = lane < kSegWindow && key < nkeys;
    int a = 0, e = 0, len = -1;  // lanes without a key rank after every real one
    if (real) {
        const int lo = offs[key], hi = offs[key + 1];
        a = j == 0 ? lo : first_at_or_past(gidx, lo, hi, j * cw);
        e = j == ncb - 1 ? hi : first_at_or_past(gidx, a, hi, (j + 1) * cw);
        len = e - a;
    }
    int rank = 0;
    for (int m = 0; m < kSegWindow; ++m) {
        const int lm = __builtin_amdgcn_readlane(len, m);
        rank += (lm > len) || (lm == len && m < lane);
    }
    if (real) seg[static_cast<int64_t>(j) * nkeys + w * kSegWindow + rank] = make_int4(key, a, e, 0);
}

// Segment of list position pos of block cb (seg: the int4 records above as int32s, rs its buffer
// resource; nothing past the tile: pos_ok false gives key 0 and an empty segment).
__device__ __forceinline__ void seg_load(__amdgpu_buffer_rsrc_t rs, int cb, int nkeys, int pos, bool pos_ok,
                                         int &key, int &a, int &len) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i r = __builtin_amdgcn_raw_buffer_load_b128(rs, pos_ok ? (cb * nkeys + pos) * 16 : kBufPast, 0, 0);
    key = r.x;
    a = r.y;
    len = r.z - r.y;
}

// act: the batch-major activation [B][opnd_rows] (fp32 or bf16, B * opnd_rows * its size < 2^31),
// read in place; batch tile
// bt = blockIdx.y covers columns [TB bt, TB bt + TB), TB = 16 VW: each lane of a slot holds VW of
// them, and one staged operand row is TB floats (swizzled, tile_stage_rows).  Logical workgroup
// L = cb * nrb + rb (XCD-contiguous).
// VP: the values are read through perm (vals[perm[k]]): the permutation is loaded with the gather
// indices two groups ahead, the values it points at one group ahead.
template <int VW, int CH, bool VP, typename InT>
__global__ __launch_bounds__(kTileThreads) void tile_spmm_kernel(
    int nkeys, int ncb, int nrb, int cw, int keys_per_rb, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ gidx, const float *__restrict__ vals, const int32_t *__restrict__ perm, int nnz,
    const InT *__restrict__ act, int opnd_rows, int64_t B, float *__restrict__ part) {
    constexpr int SL = 4;                      // slots (keys) per wave, 16 lanes each
    constexpr int TB = 16 * VW;                // batch columns of a tile
    constexpr uint32_t kRowBytes = 4u * TB;    // one staged operand row
    // static: its address is known when compiling, so a row chunk's address is one DPP XOR
    __shared__ float4 xs4[kTileLdsRows * 4 * VW + kTileClaimBytes / 16];
    const int64_t L = xcd_block();
    if (L >= static_cast<int64_t>(ncb) * nrb) return;  // whole workgroup, before any barrier
    const int cb = static_cast<int>(L / nrb), rb = static_cast<int>(L % nrb);
    const int c0 = cb * cw, cn = min(cw, opnd_rows - c0);
    const int bt = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int j = lane & 15;                    // entry of a chunk held by this lane
    const int slot = lane >> 4;                 // the row of 16 lanes is the slot
    const int ls = lane & 15;                   // lane within the slot: batch columns [ls*VW, ls*VW + VW)
    const uint32_t lane_off = static_cast<uint32_t>(ls * VW * 4);
    const uint32_t zoff = tile_row_off<VW>(cw);
    const int k_lo = rb * keys_per_rb, k_hi = min(nkeys, k_lo + keys_per_rb);
    // group G = keys k_lo + SL*G .. +SL-1, slot s taking key k_lo + SL*G + s
    const int ngroups = (k_hi - k_lo + SL - 1) / SL;
    unsigned *claims = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(xs4) + (cw + 1) * kRowBytes);
    // the block's operand rows; rows cn..cw are zero (row cw is the zero row)
    tile_stage_rows<VW, InT>(xs4, act_rsrc(act, static_cast<int>(B) * opnd_rows), opnd_rows, bt, c0, cn, cw);
    if (threadIdx.x == 0) *claims = 0u;
    __syncthreads();
    const char *lds = reinterpret_cast<const char *>(xs4);
    float *pout = part + (static_cast<int64_t>(bt) * ncb + cb) * static_cast<int64_t>(nkeys) * TB;
    // The waves take groups from the workgroup's counter as they go, so they all work until the
    // tile is done.  A group's segments come from the table when it is claimed (D - 1 groups ahead
    // of its compute), its chunks of gather indices and values one group later (VP: the permuted
    // positions, then the values they point at one group before the compute).  Chunk loads go
    // through buffer resources: lanes past a segment load from past the buffers' end, so nothing
    // is read for them.
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz), rv = buf_rsrc(vals, nnz), rp = buf_rsrc(perm, nnz);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    auto claim = [&]() {
        unsigned g = 0;
        if (lane == 0) g = atomicAdd(claims, 1u);
        return static_cast<int>(__builtin_amdgcn_readfirstlane(g));
    };
    auto seg = [&](int G, int &key, int &a, int &len) {  // this slot's segment of group G (none past the tile)
        const int pos = k_lo + SL * G + slot;
        seg_load(rs, cb, nkeys, pos, G < ngroups && pos < k_hi, key, a, len);
    };
    auto load_chunks = [&](int a, int len, int (&gi)[CH], int (&vv)[CH]) {
        const int base = (a + j) * 4;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int off = 16 * c + j < len ? base + 64 * c : kBufPast;
            gi[c] = buf_ld(rg, off);
            vv[c] = buf_ld(VP ? rp : rv, off);
        }
    };
    auto load_vals = [&](const int (&pm)[CH], int len, int (&vv)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) vv[c] = buf_ld(rv, 16 * c + j < len ? pm[c] * 4 : kBufPast);
    };
    auto group_len = [&](int len) {
        return max(max(__builtin_amdgcn_readlane(len, 0), __builtin_amdgcn_readlane(len, 16)),
                   max(__builtin_amdgcn_readlane(len, 32), __builtin_amdgcn_readlane(len, 48)));
    };
    auto compute = [&](int G, int key, int a, int len, const int (&gi)[CH], const int (&vv)[CH]) {
        const int pos = k_lo + SL * G + slot;
        const int m = group_len(len);
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (16 * c < m) {
                const bool ok = 16 * c + j < len;
                const uint32_t off = ok ? tile_row_off<VW>(gi[c] - c0) : zoff;
                const float v = ok ? __int_as_float(vv[c]) : 0.f;
                tile_chunk<VW>(acc, off, v, m - 16 * c, lane_off, lds);
            }
        }
        for (int c = CH; 16 * c < m; ++c) {  // segments longer than the prefetched chunks
            const bool ok = 16 * c + j < len;
            const int pos = (a + 16 * c + j) * 4;
            const int gv = buf_ld(rg, pos);
            const float w = __int_as_float(buf_ld(rv, VP ? (ok ? buf_ld(rp, pos) * 4 : kBufPast) : pos));
            tile_chunk<VW>(acc, ok ? tile_row_off<VW>(gv - c0) : zoff, ok ? w : 0.f, m - 16 * c, lane_off, lds);
        }
        // every chunk register is consumed here, also those a short group skipped: without this
        // use, refilling them would wait for loads issued after them
#pragma unroll
        for (int c = 0; c < CH; ++c) asm volatile("" ::"v"(gi[c]), "v"(vv[c]));
        if (pos < k_hi) {
            typedef typename TileVec<VW>::T V;
            V r;
            if constexpr (VW == 1) r = acc[0];
            else if constexpr (VW == 2) r = make_float2(acc[0], acc[1]);
            else r = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<V *>(pout + static_cast<int64_t>(key) * TB + ls * VW) = r;
        }
    };
    // ring of claimed groups: [0] computed now, [1] next, ..., [D-1] claimed this phase.  Without
    // a permutation the chunks are loaded one group ahead; with one, the chunks (gather indices and
    // permuted positions) two groups ahead and the values they point at one ahead.  (Loading the
    // values two ahead measured slower: those scattered reads are bound by the address unit, not
    // by their latency.)
    constexpr int D = VP ? 4 : 3;
    int Gs[D], Ks[D], As[D], Ls[D];
#pragma unroll
    for (int i = 0; i < D - 1; ++i) {
        Gs[i] = claim();
        seg(Gs[i], Ks[i], As[i], Ls[i]);
    }
    auto advance = [&]() {
#pragma unroll
        for (int i = 0; i + 1 < D; ++i) {
            Gs[i] = Gs[i + 1];
            Ks[i] = Ks[i + 1];
            As[i] = As[i + 1];
            Ls[i] = Ls[i + 1];
        }
        return Gs[0] < ngroups;
    };
    if constexpr (VP) {
        // buffer sets 0..2 rotate with the groups: set (t mod 3) holds group t's gather indices g,
        // permuted positions p and values v
        int g0[CH], g1[CH], g2[CH], p0[CH], p1[CH], p2[CH], v0[CH], v1[CH], v2[CH];
        load_chunks(As[0], Ls[0], g0, p0);
        load_chunks(As[1], Ls[1], g1, p1);
        load_vals(p0, Ls[0], v0);
        // one phase: claim group [3], load the chunks of [2] and the values of [1], compute [0]
        auto phase = [&](int (&gc)[CH], int (&vc)[CH], int (&pv)[CH], int (&vv)[CH], int (&gl)[CH], int (&pl)[CH]) {
            Gs[D - 1] = claim();
            seg(Gs[D - 1], Ks[D - 1], As[D - 1], Ls[D - 1]);
            load_chunks(As[2], Ls[2], gl, pl);
            load_vals(pv, Ls[1], vv);
            compute(Gs[0], Ks[0], As[0], Ls[0], gc, vc);
            return advance();
        };
        if (Gs[0] < ngroups) {
            for (;;) {
                if (!phase(g0, v0, p1, v1, g2, p2)) break;
                if (!phase(g1, v1, p2, v2, g0, p0)) break;
                if (!phase(g2, v2, p0, v0, g1, p1)) break;
            }
        }
    } else {
        int gA[CH], gB[CH], vA[CH], vB[CH];
        load_chunks(As[0], Ls[0], gA, vA);
        // one phase: claim group [2], load the chunks of [1], compute [0]
        auto phase = [&](int (&gc)[CH], int (&vc)[CH], int (&gn)[CH], int (&vn)[CH]) {
            Gs[D - 1] = claim();
            seg(Gs[D - 1], Ks[D - 1], As[D - 1], Ls[D - 1]);
            load_chunks(As[1], Ls[1], gn, vn);
            compute(Gs[0], Ks[0], As[0], Ls[0], gc, vc);
            return advance();
        };
        if (Gs[0] < ngroups) {
            for (;;) {
                if (!phase(gA, vA, gB, vB)) break;
                if (!phase(gB, vB, gA, vA)) break;
            }
        }
    }
}

// Weight gradient on the same tiles: dW[k] = sum_b dY[b, row_k] X[b, col_k] for the entries of the
// workgroup's (rows x column block) tile, with the block of X^T staged in LDS as above.  Slot s of
// a group takes row 4g + s; each lane holds its 4 batch columns of that row's dY slice and, per
// step, the dot product of its 4 columns with the entry's staged X row.  After a chunk of 16 steps
// a reduce-scatter over the slot's 16 lanes leaves lane j with entry j's sum, stored in triple
// order (16 consecutive entries per slot).  Each lane holds VW columns of a TB = 16 VW column batch
// tile (float4 at 64 columns); batch tiles are taken in turn (the block staged again), and tiles
// after the first add into dW; each entry belongs to one workgroup.
// Dot products of steps T0..T0+3: p[T0+u] = this lane's VW columns of entry T0+u's staged row
// times its VW columns of the slot's dY row.
template <int VW, int T0>
__device__ __forceinline__ void tile_dots4(float (&p)[16], const typename TileVec<VW>::T (&x)[4],
                                           const typename TileVec<VW>::T &dy) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float d = vget(x[u], 0) * vget(dy, 0);
#pragma unroll
        for (int i = 1; i < VW; ++i) d = fmaf(vget(x[u], i), vget(dy, i), d);
        p[T0 + u] = d;
    }
}

// The 16 (or nst) dot products of one chunk, four steps at a time (its 16 products and the slot's
// dY slice leave no room for a second group of reads in flight).
template <int VW>
__device__ __forceinline__ void tile_dot_chunk(float (&p)[16], uint32_t off, int nst, uint32_t lane_off,
                                               const char *lds, const typename TileVec<VW>::T &dy) {
    typedef typename TileVec<VW>::T V;
    V a[4];
    tile_reads4<VW, 0>(a, off, lane_off, lds);
    tile_dots4<VW, 0>(p, a, dy);
    if (nst > 4) {
        tile_reads4<VW, 4>(a, off, lane_off, lds);
        tile_dots4<VW, 4>(p, a, dy);
    }
    if (nst > 8) {
        tile_reads4<VW, 8>(a, off, lane_off, lds);
        tile_dots4<VW, 8>(p, a, dy);
    }
    if (nst > 12) {
        tile_reads4<VW, 12>(a, off, lane_off, lds);
        tile_dots4<VW, 12>(p, a, dy);
    }
}

// x: the batch-major X [B][opnd_rows], dy_act: the batch-major dY [B][nkeys] (fp32 or bf16), both
// read in place: the X block is staged as in tile_spmm_kernel, and each lane loads its VW batch
// columns of its slot's dY row (zero past the batch).  B * max(opnd_rows, nkeys) * the element
// size < 2^31 (32-bit buffer offsets).
template <int VW, int CH, typename InT>
__global__ __launch_bounds__(kTileThreads) void tile_sddmm_kernel(
    int nkeys, int ncb, int nrb, int cw, int keys_per_rb, int nbt, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ gidx, int nnz, const InT *__restrict__ x, int opnd_rows,
    const InT *__restrict__ dy_act, int64_t B, float *__restrict__ dw) {
    constexpr int SL = 4;
    constexpr int TB = 16 * VW;
    constexpr uint32_t kRowBytes = 4u * TB;
    typedef typename TileVec<VW>::T V;
    // static: its address is known when compiling, so a row chunk's address is one DPP XOR
    __shared__ float4 xs4[kTileLdsRows * 4 * VW + kTileClaimBytes / 16];
    const int64_t L = xcd_block();
    if (L >= static_cast<int64_t>(ncb) * nrb) return;  // whole workgroup, before any barrier
    const int cb = static_cast<int>(L / nrb), rb = static_cast<int>(L % nrb);
    const int c0 = cb * cw, cn = min(cw, opnd_rows - c0);
    const int lane = threadIdx.x & (kWave - 1);
    const int j = lane & 15;
    const int slot = lane >> 4;
    const uint32_t lane_off = static_cast<uint32_t>(j * VW * 4);
    const uint32_t zoff = tile_row_off<VW>(cw);
    const int k_lo = rb * keys_per_rb, k_hi = min(nkeys, k_lo + keys_per_rb);
    // group G = rows k_lo + SL*G .. +SL-1, taken from the workgroup's counter as in tile_spmm_kernel
    const int ngroups = (k_hi - k_lo + SL - 1) / SL;
    unsigned *claims = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(xs4) + (cw + 1) * kRowBytes);
    const char *lds = reinterpret_cast<const char *>(xs4);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    const __amdgpu_buffer_rsrc_t rx = act_rsrc(x, static_cast<int>(B) * opnd_rows);
    const __amdgpu_buffer_rsrc_t rdy = act_rsrc(dy_act, static_cast<int>(B) * nkeys);
    auto claim = [&]() {
        unsigned g = 0;
        if (lane == 0) g = atomicAdd(claims, 1u);
        return static_cast<int>(__builtin_amdgcn_readfirstlane(g));
    };
    auto seg = [&](int G, int &key, int &a, int &len) {  // this slot's segment of group G (none past the tile)
        const int pos = k_lo + SL * G + slot;
        seg_load(rs, cb, nkeys, pos, G < ngroups && pos < k_hi, key, a, len);
    };
    for (int bt = 0; bt < nbt; ++bt) {
        if (bt > 0) __syncthreads();  // the previous batch tile's reads of the block (and claims) are done
        tile_stage_rows<VW, InT>(xs4, rx, opnd_rows, bt, c0, cn, cw);
        if (threadIdx.x == 0) *claims = 0u;
        __syncthreads();
        // a group's chunks of gather indices and its rows' dY slices, one group after its claim
        auto load_group = [&](int key, int a, int len, int (&gi)[CH], V &dy) {
            const int base = (a + j) * 4;
#pragma unroll
            for (int c = 0; c < CH; ++c) gi[c] = buf_ld(rg, 16 * c + j < len ? base + 64 * c : kBufPast);
            float d[VW];  // batch rows >= B: past the buffer, 0
            const int off = ((TB * bt + VW * j) * nkeys + key) * static_cast<int>(sizeof(InT));
#pragma unroll
            for (int i = 0; i < VW; ++i) d[i] = act_ld<InT>(rdy, off + i * nkeys * static_cast<int>(sizeof(InT)));
            if constexpr (VW == 1) dy = d[0];
            else if constexpr (VW == 2) dy = make_float2(d[0], d[1]);
            else dy = make_float4(d[0], d[1], d[2], d[3]);
        };
        auto chunk = [&](int a, int len, int m, int c, uint32_t off, const V &dy) {
            float p[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) p[t] = 0.f;
            tile_dot_chunk<VW>(p, off, m - 16 * c, lane_off, lds, dy);
            const float r = group_reduce_scatter<16, 16>(p, j);
            if (16 * c + j < len) {
                float *d = dw + a + 16 * c + j;
                *d = bt == 0 ? r : *d + r;
            }
        };
        auto compute = [&](int a, int len, const int (&gi)[CH], const V &dy) {
            int m = max(max(__builtin_amdgcn_readlane(len, 0), __builtin_amdgcn_readlane(len, 16)),
                        max(__builtin_amdgcn_readlane(len, 32), __builtin_amdgcn_readlane(len, 48)));
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (16 * c < m) {
                    const bool ok = 16 * c + j < len;
                    chunk(a, len, m, c, ok ? tile_row_off<VW>(gi[c] - c0) : zoff, dy);
                }
            }
            for (int c = CH; 16 * c < m; ++c) {  // segments longer than the prefetched chunks
                const bool ok = 16 * c + j < len;
                const int gv = buf_ld(rg, (a + 16 * c + j) * 4);
                chunk(a, len, m, c, ok ? tile_row_off<VW>(gv - c0) : zoff, dy);
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) asm volatile("" ::"v"(gi[c]));
#pragma unroll
            for (int i = 0; i < VW; ++i) asm volatile("" ::"v"(vget(dy, i)));
        };
        // ring of claimed groups: [0] computed now, [1] its loads in flight, [2] claimed this phase
        int Gs[3], Ks[3], As[3], Ls[3];
        Gs[0] = claim();
        seg(Gs[0], Ks[0], As[0], Ls[0]);
        Gs[1] = claim();
        seg(Gs[1], Ks[1], As[1], Ls[1]);
        int gA[CH], gB[CH], gC[CH];
        V dA, dB, dC;
        load_group(Ks[0], As[0], Ls[0], gA, dA);
        auto phase = [&](int (&gc)[CH], V &dc, int (&gn)[CH], V &dn) {
            Gs[2] = claim();
            seg(Gs[2], Ks[2], As[2], Ls[2]);
            load_group(Ks[1], As[1], Ls[1], gn, dn);
            compute(As[0], Ls[0], gc, dc);
            Gs[0] = Gs[1], Ks[0] = Ks[1], As[0] = As[1], Ls[0] = Ls[1];
            Gs[1] = Gs[2], Ks[1] = Ks[2], As[1] = As[2], Ls[1] = Ls[2];
            return Gs[0] < ngroups;
        };
        if (Gs[0] < ngroups) {
            for (;;) {
                if (!phase(gA, dA, gB, dB)) break;
                if (!phase(gB, dB, gC, dC)) break;
                if (!phase(gC, dC, gA, dA)) break;
            }
        }
    }
}

// Both gradients in one tiled pass over the column view (one batch tile of TB = 16 VW columns).
// The workgroup stages a block of cw rows of dY (features of the output, read in place from the
// batch-major dY and swizzled as in tile_spmm_kernel); slot s of a group walks the segment of one
// column of W (the key) and holds that column's X slice: its VW batch columns of X, read in place.
// Each step reads an entry's staged dY row once and uses it twice: dX partials += v * dY row (as
// tile_spmm_kernel), and the dot product with the X slice, which a reduce-scatter over the slot's
// 16 lanes turns into dW of 16 entries per chunk.  dW goes to the walk position, or (VP: values in
// row order) to perm of it, the same permuted position the value was read from.  The block
// partials of dX are summed by tile_sum_kernel.
template <int VW, int T0>
__device__ __forceinline__ void tile_bwd_steps4(float (&acc)[VW], float (&p)[16], uint32_t off, float v,
                                                uint32_t lane_off, const char *lds,
                                                const typename TileVec<VW>::T &xs) {
    typedef typename TileVec<VW>::T V;
    V y[4];
    tile_reads4<VW, T0>(y, off, lane_off, lds);
    const float v0 = bcast16_reg<T0 + 0, T0 == 0>(v), v1 = bcast16_reg<T0 + 1, false>(v);
    const float v2 = bcast16_reg<T0 + 2, false>(v), v3 = bcast16_reg<T0 + 3, false>(v);
#pragma unroll
    for (int i = 0; i < VW; ++i) {
        acc[i] = fmaf(v0, vget(y[0], i), acc[i]);
        acc[i] = fmaf(v1, vget(y[1], i), acc[i]);
        acc[i] = fmaf(v2, vget(y[2], i), acc[i]);
        acc[i] = fmaf(v3, vget(y[3], i), acc[i]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float d = vget(y[u], 0) * vget(xs, 0);
#pragma unroll
        for (int i = 1; i < VW; ++i) d = fmaf(vget(y[u], i), vget(xs, i), d);
        p[T0 + u] = d;
    }
}

// dy: the batch-major dY [B][opnd_rows], x: the batch-major X [B][nkeys] (fp32 or bf16; B times
// max(opnd_rows, nkeys) times the element size < 2^31), B <= TB.  Groups are claimed from the
// workgroup's counter as in tile_spmm_kernel; a group's X slices are loaded with its chunks.
template <int VW, int CH, bool VP, typename InT>
__global__ __launch_bounds__(kTileThreads) void tile_bwd_kernel(
    int nkeys, int ncb, int nrb, int cw, int keys_per_rb, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ gidx, const float *__restrict__ vals, const int32_t *__restrict__ perm, int nnz,
    const InT *__restrict__ dy, int opnd_rows, const InT *__restrict__ x, int64_t B, float *__restrict__ part,
    float *__restrict__ dw) {
    constexpr int SL = 4;
    constexpr int TB = 16 * VW;
    constexpr uint32_t kRowBytes = 4u * TB;
    constexpr int kEs = static_cast<int>(sizeof(InT));
    typedef typename TileVec<VW>::T V;
    // static: its address is known when compiling, so a row chunk's address is one DPP XOR
    __shared__ float4 xs4[kTileLdsRows * 4 * VW + kTileClaimBytes / 16];
    const int64_t L = xcd_block();
    if (L >= static_cast<int64_t>(ncb) * nrb) return;  // whole workgroup, before any barrier
    // logical workgroup L = rb * ncb + cb: the column blocks of a key range sit together on one XCD,
    // which reads that range's X slices into its L2 once (the forward's L = cb * nrb + rb stages
    // each block on fewer XCDs instead).  Measured at 10k x 10k / 95 % / B = 64 with the caches
    // flushed by a read stream: 69.0 against 70.7 us with the tile sums; warm, the same.
    const int rb = static_cast<int>(L / ncb), cb = static_cast<int>(L % ncb);
    const int c0 = cb * cw, cn = min(cw, opnd_rows - c0);
    const int lane = threadIdx.x & (kWave - 1);
    const int j = lane & 15;
    const int slot = lane >> 4;
    const uint32_t lane_off = static_cast<uint32_t>(j * VW * 4);
    const uint32_t zoff = tile_row_off<VW>(cw);
    const int k_lo = rb * keys_per_rb, k_hi = min(nkeys, k_lo + keys_per_rb);
    const int ngroups = (k_hi - k_lo + SL - 1) / SL;
    unsigned *claims = reinterpret_cast<unsigned *>(reinterpret_cast<char *>(xs4) + (cw + 1) * kRowBytes);
    // the block's rows of dY; rows cn..cw are zero (row cw is the zero row)
    tile_stage_rows<VW, InT>(xs4, act_rsrc(dy, static_cast<int>(B) * opnd_rows), opnd_rows, 0, c0, cn, cw);
    if (threadIdx.x == 0) *claims = 0u;
    __syncthreads();
    const char *lds = reinterpret_cast<const char *>(xs4);
    float *pout = part + static_cast<int64_t>(cb) * nkeys * TB;
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz), rv = buf_rsrc(vals, nnz), rp = buf_rsrc(perm, nnz);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    const __amdgpu_buffer_rsrc_t rx = act_rsrc(x, static_cast<int>(B) * nkeys);
    auto claim = [&]() {
        unsigned g = 0;
        if (lane == 0) g = atomicAdd(claims, 1u);
        return static_cast<int>(__builtin_amdgcn_readfirstlane(g));
    };
    auto seg = [&](int G, int &key, int &a, int &len) {  // this slot's segment of group G (none past the tile)
        const int pos = k_lo + SL * G + slot;
        seg_load(rs, cb, nkeys, pos, G < ngroups && pos < k_hi, key, a, len);
    };
    // a group's chunks (gather indices, and values or permuted positions) and the X slice of each
    // slot's key (batch rows VW j .. VW j + VW - 1; none for an empty segment, rows >= B read as 0)
    auto load_chunks = [&](int key, int a, int len, int (&gi)[CH], int (&vv)[CH], V &xsl) {
        const int base = (a + j) * 4;
#pragma unroll
        for (int c = 0; c < CH; ++c) {  // lanes past the segment read nothing
            const int off = 16 * c + j < len ? base + 64 * c : kBufPast;
            gi[c] = buf_ld(rg, off);
            vv[c] = buf_ld(VP ? rp : rv, off);
        }
        const int xo = len > 0 ? (VW * j * nkeys + key) * kEs : kBufPast;
        const int step = len > 0 ? nkeys * kEs : 0;
        float d[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) d[i] = act_ld<InT>(rx, xo + i * step);
        if constexpr (VW == 1) xsl = d[0];
        else if constexpr (VW == 2) xsl = make_float2(d[0], d[1]);
        else xsl = make_float4(d[0], d[1], d[2], d[3]);
    };
    auto load_vals = [&](const int (&pm)[CH], int len, int (&vv)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) vv[c] = buf_ld(rv, 16 * c + j < len ? pm[c] * 4 : kBufPast);
    };
    auto group_len = [&](int len) {
        return max(max(__builtin_amdgcn_readlane(len, 0), __builtin_amdgcn_readlane(len, 16)),
                   max(__builtin_amdgcn_readlane(len, 32), __builtin_amdgcn_readlane(len, 48)));
    };
    auto chunk = [&](float (&acc)[VW], int len, int m, int c, uint32_t off, float v, int wpos, const V &xsl) {
        float p[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) p[t] = 0.f;
        const int nst = m - 16 * c;
        tile_bwd_steps4<VW, 0>(acc, p, off, v, lane_off, lds, xsl);
        if (nst > 4) tile_bwd_steps4<VW, 4>(acc, p, off, v, lane_off, lds, xsl);
        if (nst > 8) tile_bwd_steps4<VW, 8>(acc, p, off, v, lane_off, lds, xsl);
        if (nst > 12) tile_bwd_steps4<VW, 12>(acc, p, off, v, lane_off, lds, xsl);
        const float r = group_reduce_scatter<16, 16>(p, j);
        if (16 * c + j < len) dw[wpos] = r;
    };
    auto compute = [&](int G, int key, int a, int len, const int (&gi)[CH], const int (&vv)[CH],
                       const int (&pm)[CH], const V &xsl) {
        const int pos = k_lo + SL * G + slot;
        const int m = group_len(len);
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (16 * c < m) {
                const bool ok = 16 * c + j < len;
                const uint32_t off = ok ? tile_row_off<VW>(gi[c] - c0) : zoff;
                const float v = ok ? __int_as_float(vv[c]) : 0.f;
                chunk(acc, len, m, c, off, v, VP ? pm[c] : a + 16 * c + j, xsl);
            }
        }
        for (int c = CH; 16 * c < m; ++c) {  // segments longer than the prefetched chunks
            const bool ok = 16 * c + j < len;
            const int at = (a + 16 * c + j) * 4;
            const int gv = buf_ld(rg, at);
            const int pv = VP ? buf_ld(rp, at) : a + 16 * c + j;
            const float w = __int_as_float(buf_ld(rv, ok ? pv * 4 : kBufPast));
            chunk(acc, len, m, c, ok ? tile_row_off<VW>(gv - c0) : zoff, ok ? w : 0.f, pv, xsl);
        }
        // every chunk register is consumed here, also those a short group skipped: without this
        // use, refilling them would wait for loads issued after them
#pragma unroll
        for (int c = 0; c < CH; ++c) asm volatile("" ::"v"(gi[c]), "v"(vv[c]), "v"(pm[c]));
#pragma unroll
        for (int i = 0; i < VW; ++i) asm volatile("" ::"v"(vget(xsl, i)));
        if (pos < k_hi) {
            V r;
            if constexpr (VW == 1) r = acc[0];
            else if constexpr (VW == 2) r = make_float2(acc[0], acc[1]);
            else r = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<V *>(pout + static_cast<int64_t>(key) * TB + j * VW) = r;
        }
    };
    // ring of claimed groups as in tile_spmm_kernel: without a permutation the chunks and X slices
    // are loaded one group ahead; with one, two groups ahead, and the values one ahead
    constexpr int D = VP ? 4 : 3;
    int Gs[D], Ks[D], As[D], Ls[D];
#pragma unroll
    for (int i = 0; i < D - 1; ++i) {
        Gs[i] = claim();
        seg(Gs[i], Ks[i], As[i], Ls[i]);
    }
    auto advance = [&]() {
#pragma unroll
        for (int i = 0; i + 1 < D; ++i) {
            Gs[i] = Gs[i + 1];
            Ks[i] = Ks[i + 1];
            As[i] = As[i + 1];
            Ls[i] = Ls[i + 1];
        }
        return Gs[0] < ngroups;
    };
    if constexpr (VP) {
        // buffer sets 0..2 rotate with the groups: set (t mod 3) holds group t's gather indices g,
        // permuted positions p, values v and X slices x
        int g0[CH], g1[CH], g2[CH], p0[CH], p1[CH], p2[CH], v0[CH], v1[CH], v2[CH];
        V x0, x1, x2;
        load_chunks(Ks[0], As[0], Ls[0], g0, p0, x0);
        load_chunks(Ks[1], As[1], Ls[1], g1, p1, x1);
        load_vals(p0, Ls[0], v0);
        // one phase: claim group [3], load the chunks of [2] and the values of [1], compute [0]
        auto phase = [&](int (&gc)[CH], int (&pc)[CH], int (&vc)[CH], const V &xc, int (&pv)[CH], int (&vv)[CH],
                         int (&gl)[CH], int (&pl)[CH], V &xl) {
            Gs[D - 1] = claim();
            seg(Gs[D - 1], Ks[D - 1], As[D - 1], Ls[D - 1]);
            load_chunks(Ks[2], As[2], Ls[2], gl, pl, xl);
            load_vals(pv, Ls[1], vv);
            compute(Gs[0], Ks[0], As[0], Ls[0], gc, vc, pc, xc);
            return advance();
        };
        if (Gs[0] < ngroups) {
            for (;;) {
                if (!phase(g0, p0, v0, x0, p1, v1, g2, p2, x2)) break;
                if (!phase(g1, p1, v1, x1, p2, v2, g0, p0, x0)) break;
                if (!phase(g2, p2, v2, x2, p0, v0, g1, p1, x1)) break;
            }
        }
    } else {
        int gA[CH], gB[CH], vA[CH], vB[CH];
        V xA, xB;
        load_chunks(Ks[0], As[0], Ls[0], gA, vA, xA);
        // one phase: claim group [2], load the chunks of [1], compute [0]
        auto phase = [&](int (&gc)[CH], int (&vc)[CH], const V &xc, int (&gn)[CH], int (&vn)[CH], V &xn) {
            Gs[D - 1] = claim();
            seg(Gs[D - 1], Ks[D - 1], As[D - 1], Ls[D - 1]);
            load_chunks(Ks[1], As[1], Ls[1], gn, vn, xn);
            compute(Gs[0], Ks[0], As[0], Ls[0], gc, vc, gc, xc);
            return advance();
        };
        if (Gs[0] < ngroups) {
            for (;;) {
                if (!phase(gA, vA, xA, gB, vB, xB)) break;
                if (!phase(gB, vB, xB, gA, vA, xA)) break;
            }
        }
    }
}

// out[b][key] = bias[key] + sum over blocks cb (in order) of part[bt][cb][key][b - TB bt], b < nbo.
// A workgroup adds 1024/TB keys x TB batch columns of one batch tile (one float4 per thread and
// block, up to 16 blocks' loads in flight) and writes them transposed.
template <typename OutT, int TB>
__global__ __launch_bounds__(kBlock) void tile_sum_kernel(const float *__restrict__ part, int nkeys, int ncb,
                                                          int64_t nbo, const float *__restrict__ bias,
                                                          OutT *__restrict__ out, int64_t out_ld) {
    constexpr int KW = 4 * kBlock / TB;  // keys per workgroup
    constexpr int R4 = TB / 4;           // float4s per key and block
    __shared__ float tr[KW][TB + 1];
    const int k0 = blockIdx.x * KW, bt = blockIdx.y;
    const int t = threadIdx.x;
    {
        const int kk = t / R4, qq = t % R4;  // key k0 + kk, batch columns [4 qq, 4 qq + 4)
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k0 + kk < nkeys) {
            const float4 *p = reinterpret_cast<const float4 *>(
                part + ((static_cast<int64_t>(bt) * ncb) * nkeys + k0 + kk) * TB + 4 * qq);
            const int64_t stride4 = static_cast<int64_t>(nkeys) * R4;
            for (int cb0 = 0; cb0 < ncb; cb0 += 16) {
                float4 u[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    u[i] = cb0 + i < ncb ? p[(cb0 + i) * stride4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (cb0 + i < ncb) {
                        s0.x += u[i].x;
                        s0.y += u[i].y;
                        s0.z += u[i].z;
                        s0.w += u[i].w;
                    }
                }
            }
        }
        float *row = &tr[kk][4 * qq];
        row[0] = s0.x;
        row[1] = s0.y;
        row[2] = s0.z;
        row[3] = s0.w;
    }
    __syncthreads();
    const int b = t / (KW / 4), kq = (t % (KW / 4)) * 4;  // batch row TB bt + b, keys [k0 + kq, +4)
    const int64_t bb = static_cast<int64_t>(bt) * TB + b;
    if (bb < nbo) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = k0 + kq + i;
            if (key < nkeys) store_act(out, bb * out_ld + key, tr[kq + i][b] + (bias ? bias[key] : 0.f));
        }
    }
}

// ---------------------------------------------------------------- half-precision weights on MFMA
// The stored fp32 values are rounded to bf16 (nearest even) as they are read, and the products run
// on gfx950's v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32 accumulation) over tiles of W made
// dense in LDS from the stored entries; W is never dense in HBM.  The pages name Tensor-Core
// SNACK-COO for fp16/bf16 as future work (Conclusion, Limitations, and Future Work).
//
// Gather-reduce over a view (the forward over the row order, the input gradient over the column
// view): out[b][key] = bias[key] + sum over the key's entries e of bf16(v_e) * act[b][gidx_e], as a
// product of the dense tile W_view[keys][gather indices] (MFMA operand A, rows = keys) with the
// activations (operand B, columns = batch).  A workgroup owns 64 keys x 64 batch columns (2 x 2
// MFMA blocks of 32 x 32) and a run of the segment lists' blocks (a K group); it walks each block
// in two halves of 336 gather indices (from the block's 8-aligned start): it writes the half's
// entries of its keys into a zeroed LDS slab [64 keys][336] as bf16, its 4 waves take the half's
// 16-index MFMA steps in contiguous runs (wave w steps 6w .. 6w + 5), and the written cells are
// zeroed again.  Each wave reads its steps' activation operands (8 consecutive bf16 of one batch
// row per lane) straight from the batch-major activations before the half's entries are written;
// contiguous steps make each wave read whole 128-byte lines of a batch row (interleaved steps had
// four waves fetch every line, each using a quarter, and the L1 fill rate bound the kernel).  The
// 44 KB slab lets three workgroups share a CU.  At the end the waves' partial tiles are added in
// wave order through LDS: with one K group the sum plus the bias is the output, else it goes to
// part[bt][group][key][64] and tile_sum_kernel adds the groups in order.  The result does not
// depend on timing.
// A zero of the slab times a non-finite activation gives NaN: a NaN or infinite activation
// reaches every key of its tile, as in a dense product with a masked weight.
typedef __bf16 hw_bf8 __attribute__((ext_vector_type(8)));
typedef float hw_f16 __attribute__((ext_vector_type(16)));

constexpr int kHwThreads = 256;
constexpr int kHwKeys = 64;                          // keys per workgroup: two MFMA row blocks of 32
constexpr int kHwTb = 64;                            // batch columns per workgroup: two MFMA column blocks
constexpr int kHwCols = 336;                         // slab columns: half of a block's <= 645 from an 8-aligned start
constexpr int kHwSteps = kHwCols / 16;               // MFMA steps of 16 gather indices per half
constexpr int kHwWaveSteps = (kHwSteps + 3) / 4;     // steps per wave and half
constexpr int kHwRowBytes = 2 * kHwCols + 16;        // padded: consecutive slab rows start 4 banks apart
constexpr int kHwCombineLd = kHwKeys + 1;            // floats per row of the combine buffer (bank spread)
constexpr int kHwWgTarget = 768;                     // K groups make about this many workgroups (3 per CU)
static_assert(2 * kHwCols >= 638 + 7, "two halves cover a block from its 8-aligned start");
static_assert(kHwKeys * kHwRowBytes >= 4 * 32 * kHwCombineLd * 4, "combine buffer (one column block) fits the slab");

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint16_t bf16_bits_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// segs: the view's segment lists ({key, start, end, 0} per block and list position, keys of a
// 32-key window together); act: bf16 [B][ngather], B * ngather * 2 + 2048 < 2^31, ngather a
// multiple of 8 and act 16-byte aligned (each operand load is 16 aligned bytes).  Blocks
// [bpg * z, bpg * z + bpg) for blockIdx.z = z; part: NULL (one K group: out written here) or the
// fp32 partials [gridDim.y][gridDim.z][nkeys][64].
template <bool VP, typename OutT>
__global__ __launch_bounds__(kHwThreads, 3) void hw_spmm_kernel(int nkeys, int ngather, int ncb, int cw, int bpg,
                                                               const int32_t *__restrict__ segs,
                                                               const int32_t *__restrict__ gidx,
                                                               const float *__restrict__ vals,
                                                               const int32_t *__restrict__ perm, int nnz,
                                                               const bf16_t *__restrict__ act, int64_t B,
                                                               const float *__restrict__ bias, OutT *__restrict__ out,
                                                               float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) unsigned char slab[kHwKeys * kHwRowBytes];
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int k0 = blockIdx.x * kHwKeys;
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kHwTb;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    for (int i = t; i < kHwKeys * kHwRowBytes / 16; i += kHwThreads)
        reinterpret_cast<uint4 *>(slab)[i] = make_uint4(0u, 0u, 0u, 0u);
    // entry writers: 4 threads per list position of the tile
    const int pos = k0 + t / 4, sub = t % 4;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz), rv = buf_rsrc(vals, nnz), rp = buf_rsrc(perm, nnz);
    // activation operands: lane (n = lane % 32, half = lane / 32) reads batch row b0 + 32 nb + n,
    // gather indices [base + 8 half, base + 8 half + 8) of each of its steps
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(act), static_cast<short>(0), static_cast<int>(B * ngather * 2), 0x00020000);
    const int half = lane / 32, n = lane % 32;
    int arow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t b = b0 + 32 * nb + n;
        arow[nb] = b < B ? static_cast<int>(b * ngather * 2) : kBufPast;  // rows past the batch read 0
    }
    hw_f16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    __syncthreads();
    const int cb_lo = static_cast<int>(blockIdx.z) * bpg, cb_hi = min(ncb, cb_lo + bpg);
    for (int cb = cb_lo; cb < cb_hi; ++cb) {
        const int g_lo = cb * cw, g0 = g_lo & ~7;
        const int g_hi = min(g_lo + cw, ngather);
        const v4i rec = __builtin_amdgcn_raw_buffer_load_b128(
            rs, pos < nkeys ? (cb * nkeys + pos) * 16 : kBufPast, 0, 0);
        const int e_end = pos < nkeys ? rec.z : 0;
        int ecur = rec.y + sub;  // this thread's next entry of the block (every 4th of its key's run)
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            const int hs = g0 + kHwCols * h;  // the half's first gather index
            if (hs >= g_hi) break;            // uniform: depends on the block only
            const int he = min(hs + kHwCols, g_hi);
            const int nsteps = (he - hs + 15) / 16;
            const int row_off = (rec.x - k0) * kHwRowBytes - 2 * hs;
            // this wave's activation operands for the half (issued first, used after the writes)
            hw_bf8 bq[kHwWaveSteps][2];
#pragma unroll
            for (int q = 0; q < kHwWaveSteps; ++q) {
                const int s = kHwWaveSteps * w + q;
                const int col = (hs + 16 * s + 8 * half) * 2;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int off = s < nsteps && arow[nb] != kBufPast ? arow[nb] + col : kBufPast;
                    bq[q][nb] = __builtin_bit_cast(hw_bf8, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
                }
            }
            // the half's entries of this thread: a prefix of the rest of its run (sorted by index)
            const int e_first = ecur;
            for (;;) {
                int g[4], v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = ecur + 4 * u;
                    const int off = e < e_end ? e * 4 : kBufPast;
                    g[u] = e < e_end ? buf_ld(rg, off) : 0x7FFFFFFF;
                    v[u] = buf_ld(rv, VP ? (e < e_end ? buf_ld(rp, off) * 4 : kBufPast) : off);
                }
                int n_in = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (g[u] < he) {
                        *reinterpret_cast<uint16_t *>(slab + row_off + 2 * g[u]) = bf16_bits_rne(__int_as_float(v[u]));
                        ++n_in;
                    }
                }
                ecur += 4 * n_in;
                if (n_in < 4) break;
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kHwWaveSteps; ++q) {
                const int s = kHwWaveSteps * w + q;
                if (s < nsteps) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        const hw_bf8 a = *reinterpret_cast<const hw_bf8 *>(
                            slab + (32 * mb + n) * kHwRowBytes + 2 * (16 * s + 8 * half));
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb)
                            acc[mb][nb] =
                                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[q][nb], acc[mb][nb], 0, 0, 0);
                    }
                }
            }
            __syncthreads();
            // zero the cells written above (their gather indices read again)
            for (int e0 = e_first; e0 < ecur; e0 += 16) {
                int g[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) g[u] = buf_ld(rg, e0 + 4 * u < ecur ? (e0 + 4 * u) * 4 : kBufPast);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (e0 + 4 * u < ecur) *reinterpret_cast<uint16_t *>(slab + row_off + 2 * g[u]) = 0;
            }
            __syncthreads();
        }
    }
    // the waves' partial tiles, added in wave order, one column block (32 batch columns) at a
    // time: accumulator r of lane (n, half) in block (mb, nb) is key 32 mb + 8 (r / 4) + 4 half +
    // r % 4, batch column 32 nb + n
    float *cbuf = reinterpret_cast<float *>(slab);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                cbuf[(w * 32 + n) * kHwCombineLd + 32 * mb + 8 * (r / 4) + 4 * half + r % 4] = acc[mb][nb][r];
        __syncthreads();
        if (!part) {
            const int key = t % kHwKeys;
            const float bv = bias && k0 + key < nkeys ? bias[k0 + key] : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int bc = t / kHwKeys + 4 * j;
                float s = cbuf[bc * kHwCombineLd + key];
#pragma unroll
                for (int ww = 1; ww < 4; ++ww) s += cbuf[(ww * 32 + bc) * kHwCombineLd + key];
                const int64_t b = b0 + 32 * nb + bc;
                if (k0 + key < nkeys && b < B) store_act(out, b * nkeys + k0 + key, s + bv);
            }
        } else {
            const int bc = t % 32;
            float *pp = part + (static_cast<int64_t>(blockIdx.y) * gridDim.z + blockIdx.z) * nkeys * kHwTb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int key = t / 32 + 8 * j;
                float s = cbuf[bc * kHwCombineLd + key];
#pragma unroll
                for (int ww = 1; ww < 4; ++ww) s += cbuf[(ww * 32 + bc) * kHwCombineLd + key];
                if (k0 + key < nkeys) pp[static_cast<int64_t>(k0 + key) * kHwTb + 32 * nb + bc] = s;
            }
        }
        __syncthreads();
    }
}

// Wide batches: the same gather-reduce with the densified slab shared by kHwWaves batch tiles.
// A workgroup owns 64 keys x 256 batch columns; the slab of a half block is written once by all
// threads, and wave w multiplies it by batch tile w (columns b0 + 64 w ..) over all of the half's
// steps, so the entry loads and slab writes are shared by four batch tiles and each wave keeps
// its own 64 x 64 output tile (no combine across waves).  Operand B loads run six steps ahead.
constexpr int kHwWideTb = 4 * kHwTb;                 // batch columns per workgroup
constexpr int kHwAhead = 10;                         // activation operand steps in flight per wave
constexpr int64_t kHwWideMinPerKey = 64;             // entries per key from which the wide kernel runs

template <bool VP, typename OutT>
__global__ __launch_bounds__(kHwThreads, 2) void hw_spmm_wide_kernel(int nkeys, int ngather, int ncb, int cw,
                                                                    int bpg, const int32_t *__restrict__ segs,
                                                                    const int32_t *__restrict__ gidx,
                                                                    const float *__restrict__ vals,
                                                                    const int32_t *__restrict__ perm, int nnz,
                                                                    const bf16_t *__restrict__ act, int64_t B,
                                                                    const float *__restrict__ bias,
                                                                    OutT *__restrict__ out, float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) unsigned char slab[kHwKeys * kHwRowBytes];
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int k0 = blockIdx.x * kHwKeys;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kHwWideTb + kHwTb * w;  // this wave's batch tile
    const bool active = b0 < B;                                                     // uniform per wave
    for (int i = t; i < kHwKeys * kHwRowBytes / 16; i += kHwThreads)
        reinterpret_cast<uint4 *>(slab)[i] = make_uint4(0u, 0u, 0u, 0u);
    const int pos = k0 + t / 4, sub = t % 4;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz), rv = buf_rsrc(vals, nnz), rp = buf_rsrc(perm, nnz);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(act), static_cast<short>(0), static_cast<int>(B * ngather * 2), 0x00020000);
    const int half = lane / 32, n = lane % 32;
    int arow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t b = b0 + 32 * nb + n;
        arow[nb] = b < B ? static_cast<int>(b * ngather * 2) : kBufPast;
    }
    hw_f16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    __syncthreads();
    const int cb_lo = static_cast<int>(blockIdx.z) * bpg, cb_hi = min(ncb, cb_lo + bpg);
    for (int cb = cb_lo; cb < cb_hi; ++cb) {
        const int g_lo = cb * cw, g0 = g_lo & ~7;
        const int g_hi = min(g_lo + cw, ngather);
        const v4i rec = __builtin_amdgcn_raw_buffer_load_b128(
            rs, pos < nkeys ? (cb * nkeys + pos) * 16 : kBufPast, 0, 0);
        const int e_end = pos < nkeys ? rec.z : 0;
        int ecur = rec.y + sub;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            const int hs = g0 + kHwCols * h;
            if (hs >= g_hi) break;  // uniform: depends on the block only
            const int he = min(hs + kHwCols, g_hi);
            const int nsteps = (he - hs + 15) / 16;
            const int row_off = (rec.x - k0) * kHwRowBytes - 2 * hs;
            auto bload = [&](int s, int nb) {
                const int off = active && s < nsteps && arow[nb] != kBufPast ? arow[nb] + (hs + 16 * s + 8 * half) * 2
                                                                              : kBufPast;
                return __builtin_bit_cast(hw_bf8, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
            };
            hw_bf8 bq[kHwSteps][2];
#pragma unroll
            for (int s = 0; s < kHwAhead; ++s)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) bq[s][nb] = bload(s, nb);
            const int e_first = ecur;
            for (;;) {
                int g[4], v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = ecur + 4 * u;
                    const int off = e < e_end ? e * 4 : kBufPast;
                    g[u] = e < e_end ? buf_ld(rg, off) : 0x7FFFFFFF;
                    v[u] = buf_ld(rv, VP ? (e < e_end ? buf_ld(rp, off) * 4 : kBufPast) : off);
                }
                int n_in = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (g[u] < he) {
                        *reinterpret_cast<uint16_t *>(slab + row_off + 2 * g[u]) = bf16_bits_rne(__int_as_float(v[u]));
                        ++n_in;
                    }
                }
                ecur += 4 * n_in;
                if (n_in < 4) break;
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int s = 0; s < kHwSteps; ++s) {
                    if (s + kHwAhead < kHwSteps) {
#pragma unroll
                        for (int nb = 0; nb < 2; ++nb) bq[s + kHwAhead][nb] = bload(s + kHwAhead, nb);
                    }
                    if (s < nsteps) {
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb) {
                            const hw_bf8 a = *reinterpret_cast<const hw_bf8 *>(
                                slab + (32 * mb + n) * kHwRowBytes + 2 * (16 * s + 8 * half));
#pragma unroll
                            for (int nb = 0; nb < 2; ++nb)
                                acc[mb][nb] =
                                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s][nb], acc[mb][nb], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();
            for (int e0 = e_first; e0 < ecur; e0 += 16) {
                int g[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) g[u] = buf_ld(rg, e0 + 4 * u < ecur ? (e0 + 4 * u) * 4 : kBufPast);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (e0 + 4 * u < ecur) *reinterpret_cast<uint16_t *>(slab + row_off + 2 * g[u]) = 0;
            }
            __syncthreads();
        }
    }
    // each wave's 64 x 64 tile through its quarter of the slab as fp32 [64 batch columns][65]:
    // accumulator r of lane (n, half) in block (mb, nb) is key 32 mb + 8 (r / 4) + 4 half + r % 4,
    // batch column 32 nb + n
    static_assert(kHwKeys * kHwRowBytes >= kHwThreads / kWave * kHwTb * kHwCombineLd * 4 / 2,
                  "two waves' tiles fit the slab at a time");
    float *cbuf = reinterpret_cast<float *>(slab) + (w % 2) * kHwTb * kHwCombineLd;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {  // waves 0 and 1, then 2 and 3
        if (w / 2 == pass && active) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        cbuf[(32 * nb + n) * kHwCombineLd + 32 * mb + 8 * (r / 4) + 4 * half + r % 4] = acc[mb][nb][r];
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (!part) {
                const int key = k0 + lane;  // lane = key within the tile (64 keys)
                const float bv = bias && key < nkeys ? bias[key] : 0.f;
                for (int bc = 0; bc < kHwTb; ++bc) {
                    const int64_t b = b0 + bc;
                    if (key < nkeys && b < B) store_act(out, b * nkeys + key, cbuf[bc * kHwCombineLd + lane] + bv);
                }
            } else {
                const int bt = static_cast<int>(b0 / kHwTb);
                float *pp = part + (static_cast<int64_t>(bt) * gridDim.z + blockIdx.z) * nkeys * kHwTb;
                for (int r = 0; r < kHwKeys; ++r)
                    if (k0 + r < nkeys) pp[static_cast<int64_t>(k0 + r) * kHwTb + lane] = cbuf[lane * kHwCombineLd + r];
            }
        }
        __syncthreads();
    }
}

// Weight gradient with bf16 activations on the matrix cores (batches of 256 and more).  Each
// product of two bf16 values is exact in fp32, so this is the bf16 weight gradient (fp32
// accumulation, in another order) whether or not the weights are half precision.  X and dY are
// first copied feature-major as bf16 ([features][Bp], Bp the batch rounded up to 16, zero beyond
// the batch), so that the batch, the product's reduction, is contiguous per lane.  Over the view
// whose order the values are stored in (the row order: keys = rows, gather = columns; the column
// view the reverse), a workgroup owns 64 keys (two MFMA row blocks of 32) x 256 gather indices
// (a third of a segment-list block from its 8-aligned start; wave w takes column blocks 2w and
// 2w + 1) and computes the dense 64 x 256 product over the batch with
// v_mfma_f32_32x32x16_bf16, stages it in LDS as fp32, and writes dW for the stored entries of its
// keys in those 256 indices (each entry belongs to one workgroup: no partial sums).
constexpr int kHwDwKeys = 64;
constexpr int kHwDwCols = 256;                      // a third of a block's <= 645 from an 8-aligned start
constexpr int kHwDwLd = kHwDwCols + 1;              // floats per row of the staged product
constexpr int kHwDwUnroll = 4;                      // MFMA steps whose operand loads are issued together
static_assert(3 * kHwDwCols >= 638 + 7, "three thirds cover a block from its 8-aligned start");

// in [B][F] bf16 -> out [F][Bp] bf16, zero for batch rows >= B; tiles of 64 features x 64 rows.
__global__ __launch_bounds__(kBlock) void bf16_feature_major_kernel(const bf16_t *__restrict__ in, int64_t B,
                                                                    int64_t F, int64_t Bp, bf16_t *__restrict__ out) {
    __shared__ uint16_t tile[64][65];
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * 64, b0 = static_cast<int64_t>(blockIdx.y) * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t b = b0 + ty + 4 * i, f = f0 + tx;
        tile[ty + 4 * i][tx] = (b < B && f < F) ? in[b * F + f] : static_cast<uint16_t>(0);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t f = f0 + ty + 4 * i, b = b0 + tx;
        if (f < F && b < Bp) out[f * Bp + b] = tile[tx][ty + 4 * i];
    }
}

// segs: the view's segment lists; actK [nkeys][Bp], actG [ngather][Bp] (feature-major bf16,
// (max(nkeys, ngather) + 320) * Bp * 2 < 2^31, Bp a multiple of 16); dW[e] for the view's entry e.
__global__ __launch_bounds__(kHwThreads) void hw_sddmm_kernel(int nkeys, int ngather, int ncb, int cw, int Bp,
                                                             const int32_t *__restrict__ segs,
                                                             const int32_t *__restrict__ gidx, int nnz,
                                                             const bf16_t *__restrict__ actK,
                                                             const bf16_t *__restrict__ actG, float *__restrict__ dW) {
    __shared__ float cbuf[kHwDwKeys * kHwDwLd];
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int cb = static_cast<int>(blockIdx.y) / 3, third = static_cast<int>(blockIdx.y) % 3;
    const int g_lo = cb * cw, g0 = g_lo & ~7, g_hi = min(g_lo + cw, ngather);
    const int ts = g0 + kHwDwCols * third;
    if (ts >= g_hi) return;  // whole workgroup, before any barrier
    const int te = min(ts + kHwDwCols, g_hi);
    const int k0 = blockIdx.x * kHwDwKeys;
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int half = lane / 32, n = lane % 32;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(actK), static_cast<short>(0), static_cast<int>(static_cast<int64_t>(nkeys) * Bp * 2),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rgt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(actG), static_cast<short>(0), static_cast<int>(static_cast<int64_t>(ngather) * Bp * 2),
        0x00020000);
    // operand rows: keys k0 + 32 mb + n (A), gather indices ts + 64 w + 32 nb + n (B); rows past the
    // copies' ends read 0, rows of the next third or block give products that are never read
    int ka[2], gb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        ka[i] = (k0 + 32 * i + n) * Bp * 2;
        gb[i] = (ts + 64 * w + 32 * i + n) * Bp * 2;
    }
    hw_f16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    const int nsteps = Bp / 16;
    for (int s0 = 0; s0 < nsteps; s0 += kHwDwUnroll) {
        hw_bf8 a[kHwDwUnroll][2], b[kHwDwUnroll][2];
#pragma unroll
        for (int u = 0; u < kHwDwUnroll; ++u) {
            const int col = (16 * (s0 + u) + 8 * half) * 2;
            const bool ok = s0 + u < nsteps;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[u][i] = __builtin_bit_cast(hw_bf8, __builtin_amdgcn_raw_buffer_load_b128(rk, ok ? ka[i] + col : kBufPast, 0, 0));
                b[u][i] = __builtin_bit_cast(hw_bf8, __builtin_amdgcn_raw_buffer_load_b128(rgt, ok ? gb[i] + col : kBufPast, 0, 0));
            }
        }
#pragma unroll
        for (int u = 0; u < kHwDwUnroll; ++u)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][mb], b[u][nb], acc[mb][nb], 0, 0, 0);
    }
    // the product through LDS: accumulator r of lane (n, half) in block (mb, nb) is key
    // 32 mb + 8 (r / 4) + 4 half + r % 4, gather index ts + 64 w + 32 nb + n
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                cbuf[(32 * mb + 8 * (r / 4) + 4 * half + r % 4) * kHwDwLd + 64 * w + 32 * nb + n] = acc[mb][nb][r];
    __syncthreads();
    // the tile's entries: 4 threads per list position, every 4th entry of its run with a gather
    // index in [ts, te) (a contiguous part of the run, which is sorted by index)
    const int pos = k0 + t / 4, sub = t % 4;
    if (pos >= nkeys) return;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(segs, nkeys * ncb * 4);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gidx, nnz);
    const v4i rec = __builtin_amdgcn_raw_buffer_load_b128(rs, (cb * nkeys + pos) * 16, 0, 0);
    const float *crow = cbuf + (rec.x - k0) * kHwDwLd - ts;
    for (int e0 = rec.y + sub; e0 < rec.z; e0 += 16) {
        int g[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) g[u] = e0 + 4 * u < rec.z ? buf_ld(rg, (e0 + 4 * u) * 4) : 0x7FFFFFFF;
        bool past = false;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (g[u] >= ts && g[u] < te) dW[e0 + 4 * u] = crow[g[u]];
            past = past || g[u] >= te;
        }
        if (past) break;
    }
}

// ---------------------------------------------------------------- weight gradient
// xt [I][B], dyt [O][B] feature-major fp32.  A group of BT lanes per entry; lane
// t covers batch columns t*VW + m*BT*VW (+0..VW-1).  Four steps of G entries are
// loaded before any is reduced, so each lane has several gathers in flight.
template <int BT, int VW>
__global__ __launch_bounds__(kBlock) void sddmm_kernel(int64_t nnz, int64_t steps,
                                                       const int32_t *__restrict__ rows,
                                                       const int32_t *__restrict__ cols,
                                                       const float *__restrict__ xt,
                                                       const float *__restrict__ dyt, int64_t B,
                                                       float *__restrict__ dW) {
    constexpr int G = kWave / BT;
    constexpr int U = 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT, t = lane % BT;
    const int64_t w = xcd_block() * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t kbase = w * steps * G;
    for (int64_t s = 0; s < steps; s += U) {
        if (kbase + s * G >= nnz) break;  // uniform per wave
        int64_t k[U];
        bool valid[U];
        const float *xr[U];
        const float *yr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            k[u] = kbase + (s + u) * G + g;
            valid[u] = (s + u < steps) && k[u] < nnz;
            xr[u] = xt + (valid[u] ? static_cast<int64_t>(cols[k[u]]) * B : 0);
            yr[u] = dyt + (valid[u] ? static_cast<int64_t>(rows[k[u]]) * B : 0);
        }
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = 0.f;
        if constexpr (VW == 4) {
            for (int64_t bb = 4 * t; bb < B; bb += 4 * BT) {
                float4 x[U], y[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    x[u] = valid[u] ? *reinterpret_cast<const float4 *>(xr[u] + bb) : make_float4(0.f, 0.f, 0.f, 0.f);
                    y[u] = valid[u] ? *reinterpret_cast<const float4 *>(yr[u] + bb) : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    acc[u] += x[u].x * y[u].x;
                    acc[u] += x[u].y * y[u].y;
                    acc[u] += x[u].z * y[u].z;
                    acc[u] += x[u].w * y[u].w;
                }
            }
        } else {
            for (int64_t bb = t; bb < B; bb += BT) {
                float x[U], y[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    x[u] = valid[u] ? xr[u][bb] : 0.f;
                    y[u] = valid[u] ? yr[u][bb] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u] += x[u] * y[u];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int d = BT / 2; d >= 1; d >>= 1) acc[u] += __shfl_xor(acc[u], d, kWave);
            if (valid[u] && t == 0) dW[k[u]] = acc[u];
        }
    }
}

// Largest r in [0, O) with offs[r] <= e, for 0 <= e < offs[O]: the row holding entry e.
// Wave-parallel: each round samples the interval at 64 points.
__device__ int csr_row_of(const int32_t *__restrict__ offs, int O, int e, int lane) {
    int lo = 0, hi = O;  // offs[lo] <= e < offs[hi]
    while (hi - lo > kWave) {
        const int len = hi - lo;
        const int q = lo + static_cast<int>((static_cast<int64_t>(lane) * len) >> 6);
        const int c = __popcll(__ballot(offs[q] <= e));  // a prefix of the lanes, c >= 1
        const int qa = lo + static_cast<int>((static_cast<int64_t>(c - 1) * len) >> 6);
        hi = c == kWave ? hi : lo + static_cast<int>((static_cast<int64_t>(c) * len) >> 6);
        lo = qa;
    }
    const int r = lo + lane;
    const bool le = r < hi && offs[min(r, O)] <= e;
    return lo + __popcll(__ballot(le)) - 1;
}

// As csr_row_of, trying first the 64 rows around the row that entry e would be in if
// all rows had the average length (one round of loads for near-uniform layers).
__device__ int csr_row_of_guess(const int32_t *__restrict__ offs, int O, int nnz, int e, int lane) {
    // a guess only: float arithmetic (a 64-bit integer division costs ~100 scalar instructions)
    const int g = static_cast<int>(static_cast<float>(e) * (static_cast<float>(O) *
                                                            __builtin_amdgcn_rcpf(static_cast<float>(nnz))));
    const int lo = max(0, min(g - kWave / 2, O - 1));
    const int v = offs[min(lo + lane, O)];  // offs[O] = nnz > e
    const int c = __popcll(__ballot(v <= e));
    if (c >= 1 && c < kWave) return lo + c - 1;  // offs[lo + c - 1] <= e < offs[lo + c]
    return csr_row_of(offs, O, e, lane);
}

// First index j in [lo, hi) with a[j] >= target (a ascending on [lo, hi)), or hi.
// The wave first tries the 64 entries around `guess`, then narrows the interval
// 64-fold per round of loads.  Every argument is uniform across the wave.
__device__ int wave_lower_bound(const int32_t *__restrict__ a, int lo, int hi, int target, int guess, int lane) {
    // invariant: the answer lies in [lo, hi]
    if (hi - lo > kWave) {
        const int w = min(max(guess - kWave / 2, lo), hi - kWave);
        const int c = __popcll(__ballot(a[w + lane] < target));  // a prefix of the lanes
        if (c > 0 && c < kWave) return w + c;
        if (c == 0)
            hi = w;
        else
            lo = w + kWave;
    }
    while (hi - lo > kWave) {
        const int stride = (hi - lo + kWave - 1) / kWave;
        const int j = lo + lane * stride;
        const int c = __popcll(__ballot(j < hi && a[min(j, hi - 1)] < target));
        if (c == 0) return lo;
        const int nlo = lo + (c - 1) * stride + 1;
        hi = min(hi, lo + c * stride);
        lo = nlo;
    }
    if (hi <= lo) return lo;
    const int j = lo + lane;
    return lo + __popcll(__ballot(j < hi && a[min(j, hi - 1)] < target));
}

// Both gradients in one pass over the column view (batch 4*BT*Q, Q in 1..4).
// A wave owns one input column i (with NB > 1: the column's entries whose rows lie in one
// band of rows).  The column's X slice is held in registers (lane t: float4s t, t+BT, ..
// of the feature-major X row i); each stored entry k gathers its dY row once and uses it
// twice: dX[., i] += vals[k] * dY[., row k] (accumulated as in rowwave_kernel) and
// dW[k] = <X[., i], dY[., row k]> (summed over the slot's BT lanes by DPP, written at the
// entry's row-order position).  The window holds, per entry, the dY row as a 32-bit
// float4 offset, the value and that position; lanes past the range point at dY's zero row.
//
// NB == 1: a workgroup owns 4 consecutive columns and writes dX directly.  COLV (values kept in
// column-view order): the value and dW position of column-view entry j are j itself, so both
// are read and written coalesced and col_perm is not read.
// NB == kXcds: the rows are cut into 8 bands of about nnz/8 entries each, and workgroup g
// takes band g % 8 of columns 4*(g/8) .. +3.  Under round-robin dispatch band b then runs
// on XCD b alone, walking the columns in order: the dY rows, vals and dW positions that
// XCD touches are one eighth of each, and the dW lines of a row fill within a short span
// of columns, so they are completed in L2 instead of being written back piecemeal.  Each
// wave writes its band's share of dX[., i] as a feature-major row of part[b]; a second
// kernel adds the bands in order.
template <int BT, int Q, int NB, typename OutT, bool COLV = false>
__global__ __launch_bounds__(kBlock) void colbwd_kernel(
    int64_t I, const int32_t *__restrict__ coffs, const int32_t *__restrict__ crows,
    const int32_t *__restrict__ cperm, const float *__restrict__ vals, const float *__restrict__ xt,
    const float *__restrict__ dyt, int zero_row, int64_t B, OutT *__restrict__ dX, float *__restrict__ dW,
    const int32_t *__restrict__ offs, int nnz, float *__restrict__ part, int64_t nbo) {
    constexpr int S = kWave / BT;
    constexpr int UQ = 8 / Q;                                   // gathers in flight: U*Q float4s
    constexpr int U = (S * UQ <= kWave) ? UQ : kWave / S;       // S*U divides 64
    static_assert(U <= BT, "one storing lane per entry of a slot");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int e = lane / BT, t = lane % BT;
    int64_t col;
    int band = 0;
    if constexpr (NB == 1) {
        col = xcd_block() * kWavesPerBlock + wave;
    } else {
        band = blockIdx.x % NB;
        col = static_cast<int64_t>(blockIdx.x / NB) * kWavesPerBlock + wave;
    }
    const bool cok = col < I;  // uniform per wave
    const int B4 = static_cast<int>(B / 4);
    const char *__restrict__ yb = reinterpret_cast<const char *>(dyt);  // uniform base, 32-bit offsets
    const uint32_t toff = 16u * static_cast<uint32_t>(t);
    float4 acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cok) {
        float4 xv[Q];
        const float4 *__restrict__ x4 = reinterpret_cast<const float4 *>(xt) + col * B4 + t;
#pragma unroll
        for (int q = 0; q < Q; ++q) xv[q] = x4[q * BT];
        const int zoff = zero_row * B4;
        int first = coffs[col], end = coffs[col + 1];
        if constexpr (NB > 1) {
            // rows [r0, r1) of this band: r_b = the row holding entry b*nnz/NB (r_0 = 0, r_NB = O).
            // Both boundaries, and then both ends of the column's range, are found with loads
            // issued together; a window that misses falls back to the full search.
            const int O = zero_row;
            const int e0 = static_cast<int>(static_cast<int64_t>(band) * nnz / NB);
            const int e1 = min(nnz - 1, static_cast<int>(static_cast<int64_t>(band + 1) * nnz / NB));
            const float rows_per_entry = static_cast<float>(O) * __builtin_amdgcn_rcpf(static_cast<float>(nnz));
            const int q0 = max(0, min(static_cast<int>(e0 * rows_per_entry) - kWave / 2, O - 1));
            const int q1 = max(0, min(static_cast<int>(e1 * rows_per_entry) - kWave / 2, O - 1));
            const int o0 = offs[min(q0 + lane, O)], o1 = offs[min(q1 + lane, O)];  // offs[O] = nnz
            const int c0 = __popcll(__ballot(o0 <= e0)), c1 = __popcll(__ballot(o1 <= e1));
            int r0 = c0 >= 1 && c0 < kWave ? q0 + c0 - 1 : csr_row_of(offs, O, e0, lane);
            int r1 = c1 >= 1 && c1 < kWave ? q1 + c1 - 1 : csr_row_of(offs, O, e1, lane);
            if (band == 0) r0 = 0;
            if (band == NB - 1) r1 = O;
            const int s0 = first, len = end - first;
            if (len > 0 && len <= kWave) {
                const bool in = s0 + lane < end;
                const int v = crows[min(s0 + lane, end - 1)];
                first = s0 + __popcll(__ballot(in && v < r0));
                end = s0 + __popcll(__ballot(in && v < r1));
            } else if (len > kWave) {
                // guesses: where the band's rows would start and end if the column's rows were uniform
                const float per_row = static_cast<float>(len) * __builtin_amdgcn_rcpf(static_cast<float>(O));
                const int g0 = s0 + static_cast<int>(per_row * r0), g1 = s0 + static_cast<int>(per_row * r1);
                const int w0 = min(max(g0 - kWave / 2, s0), end - kWave);
                const int w1 = min(max(g1 - kWave / 2, s0), end - kWave);
                const int v0 = crows[w0 + lane], v1 = crows[w1 + lane];
                const int n0 = __popcll(__ballot(v0 < r0)), n1 = __popcll(__ballot(v1 < r1));
                const bool ok0 = (n0 > 0 || w0 == s0) && (n0 < kWave || w0 + kWave == end);
                const bool ok1 = (n1 > 0 || w1 == s0) && (n1 < kWave || w1 + kWave == end);
                const int j0 = ok0 ? w0 + n0 : wave_lower_bound(crows, s0, end, r0, g0, lane);
                const int j1 = ok1 ? w1 + n1 : wave_lower_bound(crows, s0, end, r1, g1, lane);
                first = j0;
                end = j1;
            }
        }
        int mo = zoff, mp = 0;
        float mv = 0.f;
        if (first + lane < end) {
            mp = COLV ? first + lane : cperm[first + lane];
            mo = crows[first + lane] * B4;
            mv = vals[mp];
        }
        for (int base = first; base < end; base += kWave) {
            const int co = mo, cp = mp;
            const float cv = mv;
            const int n = min(kWave, end - base);
            const int nb = base + kWave;
            if (nb < end) {  // prefetch this wave's next chunk
                mo = zoff;
                mp = 0;
                mv = 0.f;
                if (nb + lane < end) {
                    mp = COLV ? nb + lane : cperm[nb + lane];
                    mo = crows[nb + lane] * B4;
                    mv = vals[mp];
                }
            }
            for (int h = 0; h < n; h += S * U) {
                const int sa = (h + e) << 2;
                float4 y[U][Q];
                float v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t o =
                        16u * static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sa + 4 * S * u, co)) + toff;
                    v[u] = __int_as_float(__builtin_amdgcn_ds_bpermute(sa + 4 * S * u, __float_as_int(cv)));
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        y[u][q] = *reinterpret_cast<const float4 *>(yb + (o + 16u * static_cast<uint32_t>(q * BT)));
                }
                // dW: the U dot products of a slot are reduce-scattered over its BT lanes; lane t
                // with t % (BT/U) == 0 then holds entry h + e + S*(t / (BT/U)) and stores it.  The
                // stores come after the step's last gather is used (loads and stores share one
                // completion counter, so a store issued between the gathers would make each later
                // wait also wait for that store).
                float dv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float d = 0.f;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        acc[q].x = fmaf(v[u], y[u][q].x, acc[q].x);
                        acc[q].y = fmaf(v[u], y[u][q].y, acc[q].y);
                        acc[q].z = fmaf(v[u], y[u][q].z, acc[q].z);
                        acc[q].w = fmaf(v[u], y[u][q].w, acc[q].w);
                        d = fmaf(xv[q].x, y[u][q].x, d);
                        d = fmaf(xv[q].y, y[u][q].y, d);
                        d = fmaf(xv[q].z, y[u][q].z, d);
                        d = fmaf(xv[q].w, y[u][q].w, d);
                    }
                    dv[u] = d;
                }
                {
                    constexpr int R = BT / U;
                    const float dsum = group_reduce_scatter<BT, U>(dv, t);
                    const int us = t / R;
                    const int k = __builtin_amdgcn_ds_bpermute(sa + 4 * S * us, cp);
                    if (t % R == 0 && h + us * S + e < n)
                        *reinterpret_cast<float *>(reinterpret_cast<char *>(dW) + 4u * static_cast<uint32_t>(k)) =
                            dsum;
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
        for (int d = BT; d < kWave; d <<= 1) {
            acc[q].x += __shfl_xor(acc[q].x, d, kWave);
            acc[q].y += __shfl_xor(acc[q].y, d, kWave);
            acc[q].z += __shfl_xor(acc[q].z, d, kWave);
            acc[q].w += __shfl_xor(acc[q].w, d, kWave);
        }
    }
    if (cok && e == 0) {
        if constexpr (NB == 1) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {  // nbo of the B (padded) batch columns are stored
                const int64_t b0 = 4 * static_cast<int64_t>(t + q * BT);
                if (b0 + 0 < nbo) store_act(dX, (b0 + 0) * I + col, acc[q].x);
                if (b0 + 1 < nbo) store_act(dX, (b0 + 1) * I + col, acc[q].y);
                if (b0 + 2 < nbo) store_act(dX, (b0 + 2) * I + col, acc[q].z);
                if (b0 + 3 < nbo) store_act(dX, (b0 + 3) * I + col, acc[q].w);
            }
        } else {
            float4 *__restrict__ p4 = reinterpret_cast<float4 *>(part) + (band * I + col) * B4 + t;
#pragma unroll
            for (int q = 0; q < Q; ++q) p4[q * BT] = acc[q];
        }
    }
}

// dX[b][i] = sum over the NB bands, in band order, of part[band][i][b] (feature-major
// fp32 partial sums, Bp columns per row) -> batch-major OutT for b < B.  A workgroup adds and transposes a tile of 32
// columns x 64 batch rows through LDS; its stores are runs of 32 consecutive columns.
template <int NB, typename OutT>
__global__ __launch_bounds__(kBlock) void band_sum_kernel(const float *__restrict__ part, int64_t I, int64_t Bp,
                                                          int64_t B, OutT *__restrict__ dX) {
    __shared__ float tile[kTb][kTf + 1];
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTf, b0 = static_cast<int64_t>(blockIdx.y) * kTb;
    const int tid = threadIdx.x;
    const int bq = tid % 16, cr = tid / 16;  // float4 bq of the tile's batch range, column cr and cr + 16
    const int64_t B4 = Bp / 4;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int64_t c = c0 + cr + 16 * rr;
        const int64_t b4 = b0 / 4 + bq;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < I && b4 < B4) {
            float4 v[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) v[k] = reinterpret_cast<const float4 *>(part)[(k * I + c) * B4 + b4];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                s.x += v[k].x;
                s.y += v[k].y;
                s.z += v[k].z;
                s.w += v[k].w;
            }
        }
        tile[4 * bq + 0][cr + 16 * rr] = s.x;
        tile[4 * bq + 1][cr + 16 * rr] = s.y;
        tile[4 * bq + 2][cr + 16 * rr] = s.z;
        tile[4 * bq + 3][cr + 16 * rr] = s.w;
    }
    __syncthreads();
    const int c = tid % kTf;
#pragma unroll
    for (int k = 0; k < kTb / (kBlock / kTf); ++k) {
        const int bb = tid / kTf + (kBlock / kTf) * k;
        if (c0 + c < I && b0 + bb < B) store_act(dX, (b0 + bb) * I + c0 + c, tile[bb][c]);
    }
}

// Weight gradient for batches 4*BT*Q with Q in 1..4: the rowwave mapping
// for sampled products.  A workgroup owns 4/WPR rows of W, each split over WPR
// waves; a wave keeps the row's dY slice in registers (lane t: float4s t,
// t+BT, .. of the feature-major dY row, Q of them) for the whole row, takes
// the row's entries 64 at a time with their X rows as 32-bit float4 offsets
// (the next 64 prefetched; lanes past the row's end point at X's zero row),
// gathers U entries per slot in flight and reduce-scatters each slot's U dot products over its
// BT lanes by DPP.
// ld: row stride (floats) of the feature-major copies; a batch wider than 4*BT*Q is taken in
// slices of 4*BT*Q columns (xt and dyt offset by the slice), each adding into dW (ACC) after
// the first.  ACC reads the U old dW values of a step before its gathers: loads and stores
// complete in issue order on one counter, so a read issued after the gathers would make the
// step wait for all of them before its first add.  UQ: entries per slot in flight (at most
// 64/S); the slices measured fastest with 2 (5000 x 5000 at 90 %, batch 4096: 2.07 ms with 8,
// 1.87 with 2), a single pass with 8.
template <int BT, int WPR, int Q, int UQ, bool ACC>
__global__ __launch_bounds__(kBlock) void rowsddmm_kernel(int64_t O, const int32_t *__restrict__ offs,
                                                          const int32_t *__restrict__ cols,
                                                          const float *__restrict__ xt, int zero_row,
                                                          const float *__restrict__ dyt, int64_t ld,
                                                          float *__restrict__ dW) {
    constexpr int S = kWave / BT;
    constexpr int U = (S * UQ <= kWave) ? UQ : kWave / S;  // S*U divides 64
    constexpr int KPB = kWavesPerBlock / WPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int e = lane / BT, t = lane % BT;
    const int64_t r = xcd_block() * KPB + wave / WPR;
    const int wsub = wave % WPR;
    if (r >= O) return;  // uniform per wave; no barrier follows
    const int B4 = static_cast<int>(ld / 4);
    const char *__restrict__ xb = reinterpret_cast<const char *>(xt) + 16u * static_cast<uint32_t>(t);
    const float4 *__restrict__ y4 = reinterpret_cast<const float4 *>(dyt) + r * B4 + t;
    float4 dyv[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) dyv[q] = y4[q * BT];
    const int zoff = zero_row * B4;
    const int s = offs[r], end = offs[r + 1];
    const int first = s + wsub * kWave;
    int mo = zoff;
    if (first + lane < end) mo = cols[first + lane] * B4;
    for (int base = first; base < end; base += WPR * kWave) {
        const int co = mo;
        const int n = min(kWave, end - base);
        const int nb = base + WPR * kWave;
        if (nb < end) {  // prefetch this wave's next chunk
            mo = zoff;
            if (nb + lane < end) mo = cols[nb + lane] * B4;
        }
        for (int h = 0; h < n; h += S * U) {
            const int sa = (h + e) << 2;
            // the slot's U dot products are reduce-scattered over its BT lanes: lane t with
            // t % R == 0 ends with entry h + e + S*(t / R), and the wave's stores are contiguous
            constexpr int R = BT / U;
            const int src = h + (t / R) * S + e;
            float old = 0.f;
            if constexpr (ACC) old = dW[base + min(src, n - 1)];
            float4 x[U][Q];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t o = 16u * static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sa + 4 * S * u, co));
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    x[u][q] = *reinterpret_cast<const float4 *>(xb + (o + 16u * static_cast<uint32_t>(q * BT)));
            }
            float dv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float d = 0.f;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    d = fmaf(x[u][q].x, dyv[q].x, d);
                    d = fmaf(x[u][q].y, dyv[q].y, d);
                    d = fmaf(x[u][q].z, dyv[q].z, d);
                    d = fmaf(x[u][q].w, dyv[q].w, d);
                }
                dv[u] = d;
            }
            const float dsum = group_reduce_scatter<BT, U>(dv, t);
            if (t % R == 0 && src < n) dW[base + src] = ACC ? old + dsum : dsum;
        }
    }
}

// Weight gradient for batches that are multiples of 4 (and >= 16).  A wave owns
// a range of stored entries, read 64 at a time with the next 64 prefetched;
// lanes are (slot e, lane t) with S = 64/BT slots, one entry each per step;
// lane t covers batch float4s t, t+BT, ... of the entry's feature-major X row
// (gathered, U steps in flight) and of its dY row, which is kept in registers
// while consecutive entries stay in the same row (Q = B/(4*BT) float4s per
// lane; Q == 0 means "too many to cache": reload per entry).  Each slot's BT
// lanes are summed by xor shuffles.  Row offsets are 32-bit (the
// feature-major copies are < 8 GB).
template <int BT, int Q>
__global__ __launch_bounds__(kBlock) void sddmm_wide_kernel(int64_t nnz, int64_t per_wave,
                                                            const int32_t *__restrict__ rows,
                                                            const int32_t *__restrict__ cols,
                                                            const float *__restrict__ xt,
                                                            const float *__restrict__ dyt, int64_t B,
                                                            float *__restrict__ dW) {
    constexpr int S = kWave / BT;
    constexpr int U = 4;
    constexpr int QC = Q > 0 ? Q : 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int e = lane / BT, t = lane % BT;
    const int64_t wv = xcd_block() * kWavesPerBlock + threadIdx.x / kWave;
    const int64_t k0 = wv * per_wave;
    if (k0 >= nnz) return;  // uniform per wave
    const int64_t k1 = min(k0 + per_wave, nnz);
    const int B4 = static_cast<int>(B / 4);
    const float4 *__restrict__ x4 = reinterpret_cast<const float4 *>(xt);
    const float4 *__restrict__ y4 = reinterpret_cast<const float4 *>(dyt);
    int crow = -1;          // row whose dY slice is cached
    float4 dyc[QC];
    int mr = 0, mc = 0;
    if (k0 + lane < k1) {
        mr = rows[k0 + lane];
        mc = cols[k0 + lane];
    }
    for (int64_t base = k0; base < k1; base += kWave) {
        const int cr = mr, cc = mc;
        const int n = static_cast<int>(min<int64_t>(kWave, k1 - base));
        const int64_t nb = base + kWave;
        if (nb < k1) {
            mr = 0;
            mc = 0;
            if (nb + lane < k1) {
                mr = rows[nb + lane];
                mc = cols[nb + lane];
            }
        }
        for (int h = 0; h < n; h += S * U) {
            int ro[U];
            float p[U];
            if constexpr (Q > 0) {
                float4 xv[U][QC];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int src = h + u * S + e;  // < 64 because S*U divides 64
                    const int xo = __shfl(cc, src, kWave) * B4 + t;
                    ro[u] = __shfl(cr, src, kWave);
#pragma unroll
                    for (int q = 0; q < Q; ++q) xv[u][q] = x4[xo + q * BT];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (ro[u] != crow) {  // row changed: refresh the cached dY slice
                        crow = ro[u];
#pragma unroll
                        for (int q = 0; q < Q; ++q) dyc[q] = y4[crow * B4 + t + q * BT];
                    }
                    p[u] = 0.f;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        p[u] += xv[u][q].x * dyc[q].x;
                        p[u] += xv[u][q].y * dyc[q].y;
                        p[u] += xv[u][q].z * dyc[q].z;
                        p[u] += xv[u][q].w * dyc[q].w;
                    }
                }
            } else {
                int xo[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int src = h + u * S + e;
                    xo[u] = __shfl(cc, src, kWave) * B4;
                    ro[u] = __shfl(cr, src, kWave) * B4;
                    p[u] = 0.f;
                }
                for (int q = t; q < B4; q += BT) {
                    float4 xv[U], yv[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        xv[u] = x4[xo[u] + q];
                        yv[u] = y4[ro[u] + q];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        p[u] += xv[u].x * yv[u].x;
                        p[u] += xv[u].y * yv[u].y;
                        p[u] += xv[u].z * yv[u].z;
                        p[u] += xv[u].w * yv[u].w;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u] = group_sum<BT>(p[u]);
                const int src = h + u * S + e;
                if (t == 0 && src < n) dW[base + src] = p[u];
            }
        }
    }
}

// ---------------------------------------------------------------- small-batch input gradient
// For small B*I: each workgroup owns a contiguous range of stored entries in
// row order (coalesced reads of rows, cols, vals), scatters vals[k]*dY[b,rows[k]]
// into a private LDS copy of dX ([B][I]) with LDS atomic adds, and writes the
// copy to partial[w].  dx_reduce_kernel sums the partials in workgroup order.
// Summation order inside a workgroup follows the LDS atomics, so results are
// equal to rounding but not bit-reproducible run to run.
constexpr int kScatterThreads = 1024;

template <typename InT>
__global__ __launch_bounds__(kScatterThreads) void dx_scatter_kernel(int64_t nnz, int64_t per_wg, int64_t O,
                                                                     int64_t I, int64_t B,
                                                                     const int32_t *__restrict__ rows,
                                                                     const int32_t *__restrict__ cols,
                                                                     const float *__restrict__ vals,
                                                                     const InT *__restrict__ dY,
                                                                     float *__restrict__ partial) {
    extern __shared__ float dxs[];
    const int64_t n = B * I;
    for (int64_t i = threadIdx.x; i < n; i += kScatterThreads) dxs[i] = 0.f;
    __syncthreads();
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * per_wg;
    const int64_t k1 = min(k0 + per_wg, nnz);
    constexpr int U = 4;
    for (int64_t k = k0 + threadIdx.x; k < k1; k += U * kScatterThreads) {
        int r[U], c[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kk = k + u * kScatterThreads;
            const bool ok = kk < k1;
            r[u] = ok ? rows[kk] : 0;
            c[u] = ok ? cols[kk] : 0;
            v[u] = ok ? vals[kk] : 0.f;
        }
        for (int64_t b = 0; b < B; ++b) {
            float d[U];
#pragma unroll
            for (int u = 0; u < U; ++u) d[u] = load_act(dY, b * O + r[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (k + u * kScatterThreads < k1) atomicAdd(&dxs[b * I + c[u]], v[u] * d[u]);
        }
    }
    __syncthreads();
    float *__restrict__ mine = partial + static_cast<int64_t>(blockIdx.x) * n;
    for (int64_t i = threadIdx.x; i < n; i += kScatterThreads) mine[i] = dxs[i];
}

// out[i] = sum over w of partial[w][i], w ascending within each of 16 interleaved
// slices, then the slices in order: a fixed summation order.  A workgroup covers
// 64 outputs; its 16 waves take the slices and keep 8 loads in flight each.
constexpr int kReduceThreads = 1024;
template <typename OutT>
__global__ __launch_bounds__(kReduceThreads) void dx_reduce_kernel(int64_t n, int64_t nparts,
                                                                   const float *__restrict__ partial,
                                                                   OutT *__restrict__ out) {
    constexpr int kW = kReduceThreads / kWave;  // waves per workgroup, each over every kW-th part
    __shared__ float slice_sum[kW][kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + lane;
    float s = 0.f;
    if (i < n) {
        constexpr int U = 8;
        int64_t w = wave;
        for (; w + (U - 1) * kW < nparts; w += U * kW) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = partial[(w + u * kW) * n + i];
#pragma unroll
            for (int u = 0; u < U; ++u) s += v[u];
        }
        for (; w < nparts; w += kW) s += partial[w * n + i];
    }
    slice_sum[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && i < n) {
        float tot = slice_sum[0][lane];
#pragma unroll
        for (int q = 1; q < kW; ++q) tot += slice_sum[q][lane];
        store_act(out, i, tot);
    }
}

// ---------------------------------------------------------------- batch-1 CSR stream mapping
// Batch 1: the activations are vectors, so an entry's work is one multiply
// and the path is bound by streaming the triple.  A wave owns the entries
// [e0, e1) of a fixed-size chunk of the row-sorted triple and reads only cols
// and vals (8 bytes per entry): the row of each entry is recovered from
// row_offsets, read 64 rows at a time into a window that also holds those
// rows' bias (forward) or dY values (gradients).  Eight 64-entry steps of loads
// are in flight.  A step lies inside one row unless a row ends in it; only
// then are lanes told apart by row.

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the 64 lanes, the same value in every lane (fixed order).
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// 64 rows from rb: lane l holds the end offset of row rb + l and that row's value from rv
// (bias or dY; 0 when rv is null).  Rows past O read row O - 1 / offset nnz (never used).
template <typename ValT>
__device__ __forceinline__ void csr_window(const int32_t *__restrict__ offs, int O, int rb, int lane,
                                           const ValT *__restrict__ rv, int &wend, float &wval) {
    wend = offs[min(rb + 1 + lane, O)];
    wval = rv ? load_act(rv, min(rb + lane, O - 1)) : 0.f;
}

// x staged in LDS by 1024-thread workgroups (I <= kStageMaxI): a 4-byte gather from L2
// moves a whole 64-byte line, so reading x once per workgroup saves ~16x the L2 traffic.
constexpr int kStageThreads = 1024;
constexpr int64_t kStageMaxI = 16384;

// Copies x (I <= kStageMaxI elements) into LDS as fp32; every thread of the workgroup
// takes part, issuing all of its loads before its stores (one round of latency).
template <int THREADS, typename ActT>
__device__ __forceinline__ void stage_vector(const ActT *__restrict__ x, int I, float *xs) {
    constexpr int K = static_cast<int>(kStageMaxI / THREADS);
    float v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = threadIdx.x + k * THREADS;
        v[k] = i < I ? load_act(x, i) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = threadIdx.x + k * THREADS;
        if (i < I) xs[i] = v[k];
    }
    __syncthreads();
}

// Forward, batch 1: y[r] = bias[r] + sum of the row's vals * x[cols].  Rows cut by a
// chunk edge leave their partial sum in head[w] (the chunk's first row) or tail[w] (its
// last row); fixup_kernel finishes them and the empty rows, as for segscan_kernel.
// THREADS == kStageThreads: x is read from an LDS copy (I elements).
template <typename ActT, typename OutT, int THREADS, bool VPERM = false>
__global__ __launch_bounds__(THREADS) void csr1_fwd_kernel(int O, int I, int nnz, int chunk, int nchunks,
                                                           const int32_t *__restrict__ offs,
                                                           const int32_t *__restrict__ cols,
                                                           const float *__restrict__ vals,
                                                           const int32_t *__restrict__ vperm,
                                                           const ActT *__restrict__ x,
                                                           const float *__restrict__ bias, OutT *__restrict__ y,
                                                           float *__restrict__ head, float *__restrict__ tail) {
    constexpr int U = 8;
    constexpr bool kStaged = THREADS == kStageThreads;
    extern __shared__ float xs[];
    if constexpr (kStaged) stage_vector<THREADS>(x, I, xs);
    const int lane = threadIdx.x & (kWave - 1);
    const int w = static_cast<int>(xcd_block()) * (THREADS / kWave) +
                  __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    if (w >= nchunks) return;  // uniform per wave, after the only barrier
    const int e0 = w * chunk, e1 = min(e0 + chunk, nnz);
    int r = csr_row_of_guess(offs, O, nnz, e0, lane);
    const int rfirst = r;
    int rs = __builtin_amdgcn_readfirstlane(offs[r]);  // start of row r
    int rb = r, wend;
    float wbias;
    csr_window(offs, O, rb, lane, bias, wend, wbias);
    int E = __builtin_amdgcn_readlane(wend, 0);  // end of row r
    float acc = 0.f;
    for (int s0 = e0; s0 < e1; s0 += U * kWave) {
        float p[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = s0 + u * kWave + lane;
            const int kk = min(k, e1 - 1);
            const float v = vals[VPERM ? vperm[kk] : kk];
            const int c = cols[kk];
            const float xv = kStaged ? xs[c] : load_act(x, c);
            p[u] = k < e1 ? v * xv : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * kWave;
            if (s >= e1) break;
            int from = 0;  // lanes below `from` belong to rows finished in this step
            while (E < s + kWave && E < e1) {  // row r ends inside this step
                const int cut = E - s;
                const float tot = wave_sum(acc + ((lane >= from && lane < cut) ? p[u] : 0.f));
                const float bv = readlane_f(wbias, r - rb);
                acc = 0.f;
                if (E > rs && lane == 0) {  // non-empty; empty rows are left to the fix-up
                    if (rs >= e0)
                        store_act(y, r, tot + bv);
                    else
                        head[w] = tot;
                }
                from = cut;
                rs = E;
                ++r;
                if (r - rb >= kWave) {
                    rb = r;
                    csr_window(offs, O, rb, lane, bias, wend, wbias);
                }
                E = __builtin_amdgcn_readlane(wend, r - rb);
            }
            acc += lane >= from ? p[u] : 0.f;
        }
    }
    // row r holds entry e1 - 1: complete if it started in this chunk and ends at e1
    const float tot = wave_sum(acc);
    const float bv = readlane_f(wbias, r - rb);
    if (lane == 0) {
        if (rs >= e0 && E == e1)
            store_act(y, r, tot + bv);
        else if (r == rfirst)
            head[w] = tot;
        else
            tail[w] = tot;
    }
}

// Walk of one 64-entry step for the gradients: every lane gets the dY value of its
// entry's row.  Advances (r, E, window) past the rows that end inside the step.
template <typename ActT>
__device__ __forceinline__ float csr_step_rowval(int s, int e1, int lane, int O, const int32_t *__restrict__ offs,
                                                 const ActT *__restrict__ dy, int &r, int &E, int &rb, int &wend,
                                                 float &wdy) {
    float dl = readlane_f(wdy, r - rb);
    while (E < s + kWave && E < e1) {  // row r ends inside this step
        const int cut = E - s;
        ++r;
        if (r - rb >= kWave) {
            rb = r;
            csr_window(offs, O, rb, lane, dy, wend, wdy);
        }
        E = __builtin_amdgcn_readlane(wend, r - rb);
        const float d = readlane_f(wdy, r - rb);
        dl = lane >= cut ? d : dl;
    }
    return dl;
}

// Weight gradient, batch 1: dW[k] = dY[row k] * X[cols[k]], streamed in row order.
// THREADS == kStageThreads: x is read from an LDS copy (I elements).
template <typename ActT, int THREADS>
__global__ __launch_bounds__(THREADS) void csr1_dw_kernel(int O, int I, int nnz, int chunk, int nchunks,
                                                          const int32_t *__restrict__ offs,
                                                          const int32_t *__restrict__ cols,
                                                          const ActT *__restrict__ x, const ActT *__restrict__ dy,
                                                          float *__restrict__ dW) {
    constexpr int U = 8;
    constexpr bool kStaged = THREADS == kStageThreads;
    extern __shared__ float xs[];
    if constexpr (kStaged) stage_vector<THREADS>(x, I, xs);
    const int lane = threadIdx.x & (kWave - 1);
    const int w = static_cast<int>(xcd_block()) * (THREADS / kWave) +
                  __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    if (w >= nchunks) return;  // uniform per wave, after the only barrier
    const int e0 = w * chunk, e1 = min(e0 + chunk, nnz);
    int r = csr_row_of_guess(offs, O, nnz, e0, lane);
    int rb = r, wend;
    float wdy;
    csr_window(offs, O, rb, lane, dy, wend, wdy);
    int E = __builtin_amdgcn_readlane(wend, 0);
    for (int s0 = e0; s0 < e1; s0 += U * kWave) {
        float xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cols[min(s0 + u * kWave + lane, e1 - 1)];
            xv[u] = kStaged ? xs[c] : load_act(x, c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * kWave;
            if (s >= e1) break;
            const float dl = csr_step_rowval(s, e1, lane, O, offs, dy, r, E, rb, wend, wdy);
            if (s + lane < e1) dW[s + lane] = dl * xv[u];
        }
    }
}

// Input gradient, batch 1, I <= 10240, without atomics: each of a workgroup's
// 4 waves owns a private LDS copy of dX and the rows whose first entry lies in
// its chunk.  A lane takes 4 consecutive entries per step (16-byte loads of cols
// and vals), so a step covers 256 entries; two batches of kDxSteps steps are in
// flight (a CU holds only 4 of these waves, so bytes in flight per wave set the
// rate).  A step inside one row adds vals[k] * dY[row] into the copy with plain
// reads and writes: a row's columns are distinct and a wave's LDS operations
// complete in order.  A step that crosses row ends is taken row by row.  The
// copies are then added in wave order into partial[blockIdx.x], and
// dx_reduce_kernel adds the workgroups in order: the result is deterministic.
// cols and vals must be 16-byte aligned (the plan checks).
constexpr int kPrivWaves = 4;
constexpr int64_t kPrivMaxI = 10240;  // 4 copies of dX in 160 KB of LDS
constexpr int kDxSteps = 8;           // steps of 256 entries per batch of loads

// 4 entries per lane from entry s + 4*lane, clamped to the 16-byte group at kmax (the wave's
// last group below nnz & ~3).  Every path issues the same two loads, so the compiler's
// completion counting stays exact, and loads past the wave's entries hit that one cached group
// instead of fetching the next wave's; the entries [nnz & ~3, nnz) are taken separately.
__device__ __forceinline__ void dxq_load(const int32_t *__restrict__ cols, const float *__restrict__ vals, int kmax,
                                         int s, int lane, int4 &c, float4 &v) {
    const int k = min(s + 4 * lane, kmax);
    c = *reinterpret_cast<const int4 *>(cols + k);
    v = *reinterpret_cast<const float4 *>(vals + k);
}

// Row r's entries in the step of 256 from s (lanes hold entries k0 .. k0 + 3), then the
// following rows while they start inside the step, up to entry `lim`; the row state (r, its
// start Es, end E and dY value d, and the 64-row window from rb) advances with them.
template <typename ActT>
__device__ __forceinline__ void dxq_rows(float *my, int s, int k0, const int4 &c, const float4 &v, int lim, int &r,
                                         int &rb, int &Es, int &E, float &d, int &wend, float &wdy,
                                         const int32_t *__restrict__ offs, int O, const ActT *__restrict__ dy,
                                         int lane) {
    while (true) {
        const int lo = max(Es, s), hi = min(E, lim);
        const bool p0 = k0 >= lo && k0 < hi, p1 = k0 + 1 >= lo && k0 + 1 < hi;
        const bool p2 = k0 + 2 >= lo && k0 + 2 < hi, p3 = k0 + 3 >= lo && k0 + 3 < hi;
        float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
        if (p0) t0 = my[c.x];
        if (p1) t1 = my[c.y];
        if (p2) t2 = my[c.z];
        if (p3) t3 = my[c.w];
        if (p0) my[c.x] = fmaf(v.x, d, t0);
        if (p1) my[c.y] = fmaf(v.y, d, t1);
        if (p2) my[c.z] = fmaf(v.z, d, t2);
        if (p3) my[c.w] = fmaf(v.w, d, t3);
        if (E >= s + 4 * kWave || E >= lim) break;
        Es = E;
        ++r;
        if (r - rb >= kWave) {
            rb = r;
            csr_window(offs, O, rb, lane, dy, wend, wdy);
        }
        E = __builtin_amdgcn_readlane(wend, r - rb);
        d = readlane_f(wdy, r - rb);
    }
}

template <typename ActT>
__global__ __launch_bounds__(kPrivWaves *kWave) void csr1_dxpriv_kernel(int O, int I, int nnz, int chunk, int nwaves,
                                                                       const int32_t *__restrict__ offs,
                                                                       const int32_t *__restrict__ cols,
                                                                       const float *__restrict__ vals,
                                                                       const ActT *__restrict__ dy,
                                                                       float *__restrict__ partial) {
    extern __shared__ float cp[];  // [kPrivWaves][I]
    constexpr int kThreads = kPrivWaves * kWave;
    constexpr int kStep = 4 * kWave;
    constexpr int kBatch = kDxSteps * kStep;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int w = blockIdx.x * kPrivWaves + wave;
    const int a = w * chunk, b = min(a + chunk, nnz);
    const int nnz4 = nnz & ~3;
    // The first batch is loaded from the chunk's start before anything else (the row-aligned
    // start E0 >= a is found while it is in flight; entries before E0 are not used).
    const int s00 = a & ~3;
    int4 ca[kDxSteps], cb[kDxSteps];
    float4 va[kDxSteps], vb[kDxSteps];
#pragma unroll
    for (int u = 0; u < kDxSteps; ++u) dxq_load(cols, vals, nnz4 - 4, s00 + u * kStep, lane, ca[u], va[u]);
    for (int i = threadIdx.x; i < kPrivWaves * I / 4; i += kThreads)  // 4*I floats: whole float4s
        reinterpret_cast<float4 *>(cp)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    float *my = cp + wave * I;
    if (w < nwaves) {  // uniform per wave; every wave reaches the barrier below
        // entries [E0, E1): from the first row start >= a to the first row start >= b.  Both
        // ends, and the row starting at E0, come from one 64-row window of row_offsets each
        // (loaded together) when the rows near a and b are where uniform rows would put them.
        const float rows_per_entry = static_cast<float>(O) * __builtin_amdgcn_rcpf(static_cast<float>(nnz));
        const int la = max(0, min(static_cast<int>(a * rows_per_entry) - kWave / 2, O - 1));
        const int lb = max(0, min(static_cast<int>(b * rows_per_entry) - kWave / 2, O - 1));
        const int wa = offs[min(la + lane, O)], wb = offs[min(lb + lane, O)];  // offs[O] = nnz
        const int na = __popcll(__ballot(wa <= a)), nb = __popcll(__ballot(wb <= b));
        int E0, E1 = nnz;
        const bool hit_a = na >= 1 && na < kWave;  // offs[la + na - 1] <= a < offs[la + na]
        if (hit_a) {
            const int oa = __builtin_amdgcn_readlane(wa, na - 1);
            E0 = oa == a ? a : __builtin_amdgcn_readlane(wa, na);
        } else {
            const int ra = csr_row_of(offs, O, a, lane);
            const int oa = __builtin_amdgcn_readfirstlane(offs[ra]);
            E0 = oa == a ? a : __builtin_amdgcn_readfirstlane(offs[ra + 1]);
        }
        if (b < nnz) {
            if (nb >= 1 && nb < kWave) {
                const int ob = __builtin_amdgcn_readlane(wb, nb - 1);
                E1 = ob == b ? b : __builtin_amdgcn_readlane(wb, nb);
            } else {
                const int rb1 = csr_row_of(offs, O, b, lane);
                const int ob = __builtin_amdgcn_readfirstlane(offs[rb1]);
                E1 = ob == b ? b : __builtin_amdgcn_readfirstlane(offs[rb1 + 1]);
            }
        }
        if (E0 < E1) {
            // r: the row starting at E0 (the last of several that start there), from the same
            // window when it reaches past E0
            const int cr = __popcll(__ballot(wa <= E0));
            int r = hit_a && cr < kWave ? la + cr - 1 : csr_row_of(offs, O, E0, lane);
            int rb = r, wend;
            float wdy;
            csr_window(offs, O, rb, lane, dy, wend, wdy);
            int Es = E0;  // start of row r
            int E = __builtin_amdgcn_readlane(wend, 0);
            float d = readlane_f(wdy, 0);
            const int E1m = min(E1, nnz4);  // the 16-byte loads cover [.., nnz4)
            const int kmax = min(nnz4, (E1 + 3) & ~3) - 4;
            // batch of kDxSteps steps from s0 in (c, v): the whole step in row r takes the fast path
            auto run = [&](int s0, const int4 *c, const float4 *v) {
#pragma unroll
                for (int u = 0; u < kDxSteps; ++u) {
                    const int s = s0 + u * kStep;
                    if (s < E1m) {
                        if (s >= Es && E >= s + kStep && E1m >= s + kStep) {  // the whole step is row r's
                            const float t0 = my[c[u].x], t1 = my[c[u].y], t2 = my[c[u].z], t3 = my[c[u].w];
                            my[c[u].x] = fmaf(v[u].x, d, t0);
                            my[c[u].y] = fmaf(v[u].y, d, t1);
                            my[c[u].z] = fmaf(v[u].z, d, t2);
                            my[c[u].w] = fmaf(v[u].w, d, t3);
                        } else {
                            dxq_rows(my, s, s + 4 * lane, c[u], v[u], E1m, r, rb, Es, E, d, wend, wdy, offs, O, dy,
                                     lane);
                        }
                    }
                }
                // every load of the batch is complete here on every path (a skipped step included),
                // so the next batch's loads into these registers never wait for them
#pragma unroll
                for (int u = 0; u < kDxSteps; ++u) asm volatile("" ::"v"(c[u].x), "v"(v[u].x));
            };
            // two register sets used in turn (no copies, so no wait for the batch in flight)
            for (int s0 = s00; s0 < E1m; s0 += 2 * kBatch) {
#pragma unroll
                for (int u = 0; u < kDxSteps; ++u)  // the next batch, unconditionally (clamped)
                    dxq_load(cols, vals, kmax, s0 + kBatch + u * kStep, lane, cb[u], vb[u]);
                run(s0, ca, va);
                if (s0 + kBatch >= E1m) break;
#pragma unroll
                for (int u = 0; u < kDxSteps; ++u)
                    dxq_load(cols, vals, kmax, s0 + 2 * kBatch + u * kStep, lane, ca[u], va[u]);
                run(s0 + kBatch, cb, vb);
            }
            if (E1 > E1m) {  // entries [max(E0, nnz4), E1) at the end of the arrays: at most 3
                const int s = nnz4, k0 = s + 4 * lane, last = nnz - 1;
                const int4 ct = make_int4(cols[min(k0, last)], cols[min(k0 + 1, last)], cols[min(k0 + 2, last)],
                                          cols[min(k0 + 3, last)]);
                const float4 vt = make_float4(vals[min(k0, last)], vals[min(k0 + 1, last)], vals[min(k0 + 2, last)],
                                              vals[min(k0 + 3, last)]);
                dxq_rows(my, s, k0, ct, vt, E1, r, rb, Es, E, d, wend, wdy, offs, O, dy, lane);
            }
        }
    }
    __syncthreads();
    float *__restrict__ mine = partial + static_cast<int64_t>(blockIdx.x) * I;
    if (I % 4 == 0) {  // the copies and this partial are float4-aligned
        const float4 *c4 = reinterpret_cast<const float4 *>(cp);
        const int I4 = I / 4;
        for (int i = threadIdx.x; i < I4; i += kThreads) {
            float4 t = c4[i];
#pragma unroll
            for (int q = 1; q < kPrivWaves; ++q) {
                const float4 o = c4[q * I4 + i];
                t.x += o.x;
                t.y += o.y;
                t.z += o.z;
                t.w += o.w;
            }
            reinterpret_cast<float4 *>(mine)[i] = t;
        }
    } else {
        for (int i = threadIdx.x; i < I; i += kThreads) {
            float t = cp[i];
#pragma unroll
            for (int q = 1; q < kPrivWaves; ++q) t += cp[q * I + i];
            mine[i] = t;
        }
    }
}

__global__ __launch_bounds__(kBlock) void zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------- bias gradient
template <typename InT>
__global__ __launch_bounds__(kBlock) void bias_grad_kernel(int64_t O, int64_t B, const InT *__restrict__ dY,
                                                           float *__restrict__ db) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (o >= O) return;
    float s = 0.f;
    for (int64_t b = 0; b < B; ++b) s += load_act(dY, b * O + o);
    db[o] = s;
}

// ================================================================ host side
using snack::fail;
using snack::option;

thread_local hipEvent_t g_probe_start = nullptr;
thread_local hipEvent_t g_probe_stop = nullptr;
thread_local int g_probe_mute = 0;  // > 0: a caller brackets several launches itself

// Records the armed probe's start event (before the main kernel) or stop event (after it).
inline void probe(bool start, hipStream_t st) {
    if (g_probe_mute > 0) return;
    hipEvent_t e = start ? g_probe_start : g_probe_stop;
    if (e) (void)hipEventRecord(e, st);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline int64_t round_up8(int64_t x) { return ceil_div(x, kXcds) * kXcds; }

enum Mapping { kSegscan = 0, kRowwave = 1, kScatter = 2, kCsr1 = 3, kCsr1Priv = 4, kTile = 5 };
constexpr int64_t kPrivMinNnz = int64_t(1) << 21;  // batch-1 input gradient: private copies from here
constexpr int64_t kScatterLdsFloats = 16384;  // 64 KB private dX copy per workgroup

// Device work plan of one gather-reduce (forward or input gradient).
// Batch limits of the gather-reduce mappings: the input gradient scatters into LDS copies at
// batch 1, and batches from 4 on take the rowwave mapping (tiles of 4*BT columns, or one tile of
// 4*BT*Q columns, Q <= 4, where 4*BT does not divide the padded batch).
constexpr int64_t kScatterMaxB = 1;
constexpr int64_t kRowwaveMinB = 4;

// layers from which the wide-batch gradient paths (column-order values for the input gradient,
// 256-column slices for the weight gradient) pay off over the plain ones
constexpr int64_t kLargeBatchMinNnz = int64_t(1) << 18;

struct SpmmPlan {
    Mapping mapping;
    bool cvals;          // rowwave over the column view: vals gathered into column order first
    int bt;              // batch lanes per entry group (segscan) or lanes per slot (rowwave)
    int q;               // rowwave: float4s per lane (batch tile 4*bt*q)
    int64_t chunk;       // segscan, csr1: entries per wave; scatter: entries per workgroup
    int64_t nchunks;     // segscan, csr1: waves; scatter: workgroups (partial copies)
    int64_t nparts;      // csr1 private copies: workgroups (partial copies)
    bool direct;         // operand used in place (fp32 at batch 1; the tiled walk) instead of a transposed copy
    int64_t bpad;        // batch columns of the feature-major operand (rowwave: B rounded up to 4)
    size_t off_opnd, off_head, off_tail, off_cvals, total;
    // kTile: batch columns per tile (16, 32 or 64), prefetched chunks, column blocks, key blocks,
    // block width, keys per key block, batch tiles; offset table and partial sums in the workspace
    int ttb, tch, tncb, tnrb, tcw, tkpr, tnbt, tnnz;
    size_t off_tab, off_part;
};

// Batch columns of the feature-major copies.  The float4-lane kernels take batch tiles of
// 4*BT*Q columns (BT a power of two <= 16, Q <= 4 float4s per lane); a batch up to 256 is padded
// with zero columns to the smallest such size, so one tile covers it and the backward pass runs
// fused, and a larger one to a multiple of 4.  The kernels store only the real columns; the
// padded products are exact zeros.
inline int64_t pad_batch(int64_t B) {
    if (B <= 1) return B;
    if (B <= 256) {
        constexpr int64_t kTiles[] = {4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256};
        for (int64_t t : kTiles)
            if (t >= B) return t;
    }
    return (B + 3) / 4 * 4;
}

inline int pow2_at_least(int64_t x) {
    int p = 1;
    while (p < x && p < kWave) p <<= 1;
    return p;
}

// nout = outputs per batch row; scatter_ok: the caller can run the scatter
// mapping (input gradient: row-order entries, outputs indexed by column).
// (values in column order are read from a gathered copy in the workspace, which is aligned)
bool vec16(const snack_coo_desc *W) {
    return reinterpret_cast<uintptr_t>(W->cols) % 16 == 0 &&
           (W->row_to_col || reinterpret_cast<uintptr_t>(W->vals) % 16 == 0);
}

SpmmPlan plan_spmm_map(int64_t nnz, int64_t opnd_rows, int64_t nout, int64_t B, int dtype, bool scatter_ok,
                       bool aligned16) {
    SpmmPlan p{};
    p.bpad = B;
    p.direct = (B == 1 && dtype == SNACK_F32);
    // batch 1, rows averaging >= 32 entries: stream cols and vals, rows from row_offsets,
    // activations read in place (the segmented scan is faster for shorter rows)
    if (B == 1 && !scatter_ok && nnz > 0 && nnz >= 32 * nout) {
        p.direct = true;
        p.mapping = kCsr1;
        p.chunk = round_up(ceil_div(nnz, 8192), 256);  // about 8192 waves
        p.nchunks = ceil_div(nnz, p.chunk);
        size_t at = 0;
        p.off_opnd = 0;
        p.off_head = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>(p.nchunks));
        p.off_tail = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>(p.nchunks));
        p.total = at;
        return p;
    }
    // batch-1 input gradient of a large layer: private per-wave copies of dX, no atomics
    if (B == 1 && scatter_ok && aligned16 && nnz >= kPrivMinNnz && nout <= kPrivMaxI) {
        p.direct = true;
        p.mapping = kCsr1Priv;
        // about 256 workgroups per 4 copies of dX that fit a CU's LDS, 4 waves each
        const int64_t parts = 256 * std::min<int64_t>(4, std::max<int64_t>(1, kPrivMaxI / nout));
        p.chunk = round_up(ceil_div(nnz, parts * kPrivWaves), kWave);
        p.nchunks = ceil_div(nnz, p.chunk);
        p.nparts = ceil_div(p.nchunks, kPrivWaves);
        size_t at = 0;
        p.off_opnd = 0;
        p.off_head = p.off_tail = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>(p.nparts * nout));
        p.total = at;
        return p;
    }
    if (scatter_ok && B <= kScatterMaxB && B * nout <= kScatterLdsFloats && nnz > 0) {
        p.mapping = kScatter;
        p.direct = true;  // reads dY in its batch-major layout
        p.nchunks = std::min<int64_t>(std::max<int64_t>(ceil_div(nnz, 4096), 1), 256);
        p.chunk = ceil_div(nnz, p.nchunks);
        size_t at = 0;
        p.off_opnd = p.off_tail = 0;
        p.off_head = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>(p.nchunks * B * nout));
        p.total = at;
        return p;
    }
    const int64_t Bp = pad_batch(B);
    p.bpad = B;
    if (Bp >= kRowwaveMinB && (opnd_rows + 1) * Bp * 4 < (int64_t(1) << 32)) {
        p.mapping = kRowwave;
        p.bpad = Bp;
        p.bt = 1;  // lanes per slot: the largest power of two <= min(16, Bp/4)
        while (p.bt * 2 <= std::min<int64_t>(16, Bp / 4)) p.bt *= 2;
        p.q = 1;
        if (Bp % (4 * p.bt) != 0) {
            // one exact tile of 4*BT*Q columns, Q <= 4 float4s per lane, where one exists
            for (int bt = 16; bt >= 1; bt /= 2) {
                if (Bp % (4 * bt) == 0 && Bp / (4 * bt) <= 4) {
                    p.bt = bt;
                    p.q = static_cast<int>(Bp / (4 * bt));
                    break;
                }
            }
        } else if (Bp % 256 == 0 && nnz < 16 * nout) {
            // keys averaging < 16 entries at wide batches: 256-column tiles (4 float4s per lane), so
            // each key's index loads serve 4x the columns (a wave per key is latency-bound there)
            p.bt = 16;
            p.q = 4;
        }
    } else {
        p.mapping = kSegscan;
        p.bt = pow2_at_least(B);
        const int64_t G = kWave / p.bt;
        const int64_t target_waves = 8192;
        int64_t steps = ceil_div(std::max<int64_t>(nnz, 1), G * target_waves);
        steps = std::min<int64_t>(std::max<int64_t>(steps, 2), 32);
        p.chunk = G * steps;
        p.nchunks = ceil_div(nnz, p.chunk);
    }
    size_t at = 0;
    p.off_opnd = at;
    if (!p.direct) at = align_up(at + sizeof(float) * static_cast<size_t>((opnd_rows + 1) * p.bpad));
    p.off_head = at;
    if (p.mapping == kSegscan) at = align_up(at + sizeof(float) * static_cast<size_t>(p.nchunks * B));
    p.off_tail = at;
    if (p.mapping == kSegscan) at = align_up(at + sizeof(float) * static_cast<size_t>(p.nchunks * B));
    p.total = at;
    return p;
}

// The LDS-tiled gather-reduce (kTile) for batches padded to a multiple of 16 on layers of at
// least kTileMinNnz entries whose segments per (key, block) average at least 8 entries; the batch
// tile is 64 columns where the padded batch allows, else 32 or 16.  SNACK_COO_TILE=0 in the
// environment turns the tiled kernels off.
constexpr int64_t kTileMinNnz = int64_t(1) << 20;
// Up to 64 batch tiles (4096 columns): each tile walks the entries again over its own staged
// columns, and the block partials grow with the batch (4096 x 8 blocks x 5000 keys: 655 MB on the
// 5000 x 5000 layer), which 288 GB of HBM holds; the wide-batch gather paths measured 1.6x slower
// there (5.65 against 3.47 ms per step at 90 %).  Wider batches keep the gather paths.
constexpr int64_t kTileMaxBatchTiles = 64;

int tile_env() { return option(SNACK_OPT_TILE) == 0 ? 0 : -1; }

// Column blocks over n operand rows: ncb = ceil(n / kTileMaxCols) blocks of cw = ceil(n / ncb)
// (the layout of snack_coo_desc.row_blocks / col_blocks; one block for n = 0).
void tile_blocks(int64_t n, int64_t &ncb, int64_t &cw) {
    ncb = std::max<int64_t>(1, ceil_div(n, kTileMaxCols));
    cw = std::max<int64_t>(1, ceil_div(n, ncb));
}

// Keys per key range of the tiled walks: about 256 workgroups in all (one per CU at 64 columns,
// two at 16 or 32), at most one key per thread of a 1024-thread workgroup.
int tile_keys_per_range(int64_t nkeys, int64_t ncb, int tb) {
    const int64_t per_cu = tb == 64 ? 1 : 2;
    const int64_t nrb0 = std::max<int64_t>(1, ceil_div(256 * per_cu, ncb));
    return static_cast<int>(std::min<int64_t>(ceil_div(nkeys, nrb0), kTileWaves * kWave));
}

void plan_tile(SpmmPlan &p, int64_t nnz, int64_t opnd_rows, int64_t nkeys, int64_t B) {
    const int env = tile_env();
    if (env == 0) return;
    const int64_t Bp = pad_batch(B);
    const int tb = Bp % 64 == 0 ? 64 : (Bp % 32 == 0 ? 32 : (Bp % 16 == 0 ? 16 : 0));
    // nnz < 2^29: the tiles read the per-entry arrays (and the segment table) through 32-bit byte
    // offsets, which stay below 2^31 and below the out-of-range offset kBufPast.  At most
    // kTileMaxBatchTiles batch tiles.
    // The operand is read through 32-bit byte offsets too: Bp * opnd_rows floats below 2^31 bytes.
    if (tb == 0 || Bp / tb > kTileMaxBatchTiles || nnz < kTileMinNnz || nnz >= (int64_t(1) << 29) ||
        opnd_rows < 1 || nkeys < 1 || Bp * opnd_rows >= (int64_t(1) << 29))
        return;
    int64_t ncb, cw;
    tile_blocks(opnd_rows, ncb, cw);
    const double mean = static_cast<double>(nnz) / static_cast<double>(nkeys * ncb);
    if (mean < 8.0 || nkeys * ncb * 4 >= (int64_t(1) << 29)) return;
    p.mapping = kTile;
    p.bpad = Bp;
    p.ttb = tb;
    p.tnnz = static_cast<int>(nnz);
    const double need = mean + 4.0 * std::sqrt(mean) + 1.0;
    p.tch = need <= 32.0 ? 2 : (need <= 64.0 ? 4 : 8);
    p.tncb = static_cast<int>(ncb);
    p.tcw = static_cast<int>(cw);
    p.tkpr = tile_keys_per_range(nkeys, ncb, tb);
    p.tnrb = static_cast<int>(ceil_div(nkeys, p.tkpr));
    p.tnbt = static_cast<int>(Bp / tb);
    p.direct = true;  // the tiles stage their blocks from the batch-major activation
    size_t at = 0;
    p.off_opnd = at;
    p.off_tab = at;
    at = align_up(at + 4 * sizeof(int32_t) * static_cast<size_t>(nkeys * ncb));
    p.off_part = at;
    at = align_up(at + sizeof(float) * static_cast<size_t>(Bp) * static_cast<size_t>(ncb) *
                           static_cast<size_t>(nkeys));
    p.off_head = p.off_tail = at;
    p.total = at;
}

// Appends n floats of workspace for values gathered into the order of the walk (off_cvals).
void add_cvals(SpmmPlan &p, int64_t n) {
    p.cvals = true;
    p.off_cvals = align_up(p.total);
    p.total = align_up(p.off_cvals + sizeof(float) * static_cast<size_t>(n));
}

// aligned16: cols and vals are 16-byte aligned (the batch-1 private-copy kernel loads 4 entries at once).
// colvals: the values are stored in column-view order (snack_coo_desc.row_to_col != NULL).
SpmmPlan plan_spmm(int64_t nnz, int64_t opnd_rows, int64_t nout, int64_t B, int dtype, bool scatter_ok,
                   bool aligned16 = false, bool colvals = false) {
    // with values in column order the input gradient (scatter_ok) walks only the column view, where
    // they are in place: the batch-1 CSR walk of the forward serves it there, and the row walks
    // (private copies, scatter) are not used
    // Below kPrivMinNnz entries the batch-1 input gradient walks the column view whatever the value
    // order (values in row order read through col_perm), as the forward walks the rows: measured on
    // 10k x 10k layers, 11.2 against 18.9 us at 99 % and 6.9 against 11.1 us at 99.9 % for the LDS
    // scatter and its reduce.  Above it the permuted reads cost more than the private copies of dX
    // (38 against 23 us at 95 %).
    const bool b1_col = B == 1 && nnz < kPrivMinNnz;
    SpmmPlan p = plan_spmm_map(nnz, opnd_rows, nout, B, dtype, scatter_ok && !colvals && !b1_col, aligned16);
    // the LDS-tiled walk where it applies (values in the walk's order, or read through the
    // permutation: the input gradient with values in row order, the forward in column order)
    if (p.mapping == kRowwave) plan_tile(p, nnz, opnd_rows, nout, B);
    if (p.mapping == kTile && scatter_ok != colvals && p.tnbt >= 4) add_cvals(p, nnz);
    // the rowwave walks read the values through a permutation -- the input gradient with values in
    // row order, the forward with values in column order -- once per batch tile; with 4 or more
    // tiles on a large layer they are gathered into the walk's order once, so every tile reads them
    // coalesced (one tile: the gather costs more than it saves)
    if (scatter_ok != colvals && p.mapping == kRowwave && ceil_div(p.bpad, 4 * p.bt * p.q) >= 4 &&
        nnz >= kLargeBatchMinNnz)
        add_cvals(p, nnz);
    return p;
}

struct SddmmPlan {
    bool csr1;           // batch 1: csr1_dw_kernel, activations read in place
    bool wide;           // sddmm_wide_kernel (batch a multiple of 4, >= 16) or sddmm_kernel
    int rowq;            // > 0: rowsddmm_kernel with this many float4s per lane (1 to 4)
    int64_t slices;      // rowsddmm over this many 256-column batch slices (1: the whole batch)
    int bt, vw;
    int64_t steps, waves, per_wave;
    bool x_direct, dy_direct;
    int64_t bpad;        // batch columns of the feature-major copies (rowsddmm: B rounded up to 4)
    size_t off_dw;       // row-order dW staging (values in column order)
    size_t off_x, off_dy, total;
    // LDS-tiled weight gradient (tile_sddmm_kernel): batch columns per tile (16, 32 or 64),
    // chunks, column blocks, key blocks, block width, keys per key block, batch tiles; segment
    // table in the workspace
    bool tile;
    int ttb, tch, tncb, tnrb, tcw, tkpr, tnbt, tnnz;
    size_t off_tab;
};

// colvals: dW goes out in column-view order; the kernels write it in row order to the
// workspace (off_dw) and a gather through col_perm reorders it.
SddmmPlan plan_sddmm(int64_t nnz, int64_t O, int64_t I, int64_t B, int dtype, bool colvals = false) {
    SddmmPlan p{};
    const int64_t target_waves = 8192;
    if (B >= 16 && B % 4 == 0) {
        p.wide = true;
        p.bt = 4;  // lanes per entry: the largest power of two <= min(16, B/4)
        while (p.bt * 2 <= std::min<int64_t>(16, B / 4)) p.bt *= 2;
        p.per_wave = std::min<int64_t>(256, ceil_div(ceil_div(std::max<int64_t>(nnz, 1), target_waves), kWave) * kWave);
        p.waves = ceil_div(nnz, p.per_wave);
    } else {
        p.wide = false;
        p.vw = (B % 4 == 0) ? 4 : 1;
        // about 16 batch columns per lane before the cross-lane reduction
        int64_t bt = std::max<int64_t>(1, B / 16);
        int b2 = 1;
        while (b2 * 2 <= bt && b2 < 16) b2 <<= 1;
        p.bt = b2;
        const int64_t G = kWave / p.bt;
        p.steps = std::min<int64_t>(std::max<int64_t>(ceil_div(std::max<int64_t>(nnz, 1), G * target_waves), 1), 64);
        p.waves = ceil_div(nnz, G * p.steps);
    }
    p.slices = 1;
    p.bpad = B;
    const int64_t Bp = pad_batch(B);
    if (Bp >= 4 && (std::max(I, O) + 1) * Bp * 4 < (int64_t(1) << 32)) {
        // rowsddmm over the padded batch Bp = 4*BT*Q: BT the largest power of two <= 16 that
        // leaves Q <= 4
        for (int bt = 16; bt >= 1; bt /= 2) {
            if (Bp % (4 * bt) == 0 && Bp / (4 * bt) <= 4) {
                p.bt = bt;
                p.rowq = static_cast<int>(Bp / (4 * bt));
                break;
            }
        }
        // wide batch, large layer or rows averaging < 16 entries:
        if (p.rowq == 0 && Bp % 256 == 0 && (nnz >= kLargeBatchMinNnz || nnz < 16 * O)) {
            // slices of 256 columns (each gathers its part of the X rows once per entry; the
            // per-entry kernel re-reads the whole dY row per entry)
            p.bt = 16;
            p.rowq = 4;
            p.slices = Bp / 256;
        }
        if (p.rowq > 0) p.bpad = Bp;
    }
    p.x_direct = p.dy_direct = (B == 1 && dtype == SNACK_F32);
    // rows averaging >= 128 entries; with values in column order the walk is over the column view
    // (columns averaging >= 128 entries), which writes dW in that order directly
    if (B == 1 && nnz >= 128 * (colvals ? I : O)) {
        p.csr1 = true;
        p.x_direct = p.dy_direct = true;
        p.steps = round_up(ceil_div(std::max<int64_t>(nnz, 1), 8192), 256);  // entries per wave
        p.waves = ceil_div(nnz, p.steps);
    }
    // the LDS-tiled walk: batches padded to a multiple of 64 on large layers whose (row, column
    // block) segments average at least 8 entries
    const int tb = Bp % 64 == 0 ? 64 : (Bp % 32 == 0 ? 32 : (Bp % 16 == 0 ? 16 : 0));
    if (!p.csr1 && tile_env() != 0 && tb > 0 && Bp / tb <= kTileMaxBatchTiles && nnz >= kTileMinNnz &&
        nnz < (int64_t(1) << 29) && I > 0 && O > 0 && Bp * std::max(I, O) < (int64_t(1) << 29)) {
        int64_t ncb, cw;
        tile_blocks(I, ncb, cw);
        const double mean = static_cast<double>(nnz) / static_cast<double>(O * ncb);
        if (mean >= 8.0 && O * ncb * 4 < (int64_t(1) << 29)) {
            p.tile = true;
            p.ttb = tb;
            p.tnnz = static_cast<int>(nnz);
            p.rowq = 0;
            p.slices = 1;
            p.bpad = Bp;
            p.x_direct = p.dy_direct = true;  // X staged and dY read in their batch-major layout
            const double need = mean + 4.0 * std::sqrt(mean) + 1.0;
            // 8 chunks at 64 columns would spill registers; longer segments take their further
            // chunks unprefetched there
            p.tch = need <= 32.0 ? 2 : (need <= 64.0 || tb == 64 ? 4 : 8);
            p.tncb = static_cast<int>(ncb);
            p.tcw = static_cast<int>(cw);
            p.tkpr = tile_keys_per_range(O, ncb, tb);
            p.tnrb = static_cast<int>(ceil_div(O, p.tkpr));
            p.tnbt = static_cast<int>(Bp / tb);
        }
    }
    size_t at = 0;
    p.off_x = at;
    if (!p.x_direct) at = align_up(at + sizeof(float) * static_cast<size_t>((I + 1) * p.bpad));
    p.off_dy = at;
    if (!p.dy_direct) at = align_up(at + sizeof(float) * static_cast<size_t>((O + 1) * p.bpad));
    p.off_dw = at;
    if (colvals && nnz > 0 && !p.csr1) at = align_up(at + sizeof(float) * static_cast<size_t>(nnz));
    p.off_tab = at;
    if (p.tile) at = align_up(at + 4 * sizeof(int32_t) * static_cast<size_t>(O * p.tncb));
    p.total = at;
    return p;
}

int check_hip(const char *what);
int launch_bounds(int64_t nkeys, int ncb, int cw, const int32_t *offs, const int32_t *gidx, int32_t *tab,
                  hipStream_t st);

// Allows kernel (name, f) lds bytes of dynamic LDS -- the most any of its launches asks for --
// once per device: done holds a bit per device already set.
int allow_lds(const void *f, size_t lds, std::atomic<uint64_t> &done, const char *name) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return check_hip(name);
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return SNACK_OK;
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return fail(SNACK_ERR_HIP, "%s: %zu bytes of LDS: %s", name, lds, hipGetErrorString(e));
    done.fetch_or(bit, std::memory_order_release);
    return SNACK_OK;
}

template <int VW, int CH, typename InT>
int launch_tile_sddmm_kernel(const SddmmPlan &p, int64_t O, int64_t I, int64_t B, const int32_t *tab,
                             const int32_t *cols, const InT *X, const InT *dY, float *dw, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(round_up8(static_cast<int64_t>(p.tncb) * p.tnrb)));
    hipLaunchKernelGGL((tile_sddmm_kernel<VW, CH, InT>), grid, dim3(kTileThreads), 0, st, static_cast<int>(O),
                       p.tncb, p.tnrb, p.tcw, p.tkpr, p.tnbt, tab, cols, p.tnnz, X, static_cast<int>(I), dY, B, dw);
    return check_hip("tile_sddmm_kernel");
}

template <typename InT>
int launch_tile_sddmm_t(const SddmmPlan &p, int64_t O, int64_t I, int64_t B, const int32_t *tab,
                        const int32_t *cols, const InT *X, const InT *dY, float *dw, hipStream_t st) {
    // 8 prefetched chunks only below 64 columns (at 64 they would spill registers)
    switch (p.ttb * 16 + std::min(p.tch, p.ttb == 64 ? 4 : 8)) {
        case 16 * 16 + 2: return launch_tile_sddmm_kernel<1, 2>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 16 * 16 + 4: return launch_tile_sddmm_kernel<1, 4>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 16 * 16 + 8: return launch_tile_sddmm_kernel<1, 8>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 32 * 16 + 2: return launch_tile_sddmm_kernel<2, 2>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 32 * 16 + 4: return launch_tile_sddmm_kernel<2, 4>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 32 * 16 + 8: return launch_tile_sddmm_kernel<2, 8>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 64 * 16 + 2: return launch_tile_sddmm_kernel<4, 2>(p, O, I, B, tab, cols, X, dY, dw, st);
        case 64 * 16 + 4: return launch_tile_sddmm_kernel<4, 4>(p, O, I, B, tab, cols, X, dY, dw, st);
        default: return fail(SNACK_ERR_INTERNAL, "tile: unsupported plan (batch tile %d, chunks %d)", p.ttb, p.tch);
    }
}

// The tiled weight gradient (row view): segment table (unless the layer has one), then the tiles,
// which read X and dY (act_dtype) in their batch-major layout.
int launch_tile_sddmm(const SddmmPlan &p, const snack_coo_desc *W, const void *X, const void *dY, int64_t B,
                      int act_dtype, float *dw, int32_t *tab_ws, hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features;
    const int32_t *tab = W->row_blocks;
    probe(true, st);
    if (!tab) {
        int32_t *t = tab_ws;
        if (int s = launch_bounds(O, p.tncb, p.tcw, W->row_offsets, W->cols, t, st)) return s;
        tab = t;
    }
    const int s = act_dtype == SNACK_F32
                      ? launch_tile_sddmm_t(p, O, I, B, tab, W->cols, static_cast<const float *>(X),
                                            static_cast<const float *>(dY), dw, st)
                      : launch_tile_sddmm_t(p, O, I, B, tab, W->cols, static_cast<const bf16_t *>(X),
                                            static_cast<const bf16_t *>(dY), dw, st);
    probe(false, st);
    return s;
}

// Backward pass plan: the fused column-view kernel for (padded) batches 4*BT*Q (Q in 1..4)
// whose feature-major copies (with their zero rows) stay below 4 GB; otherwise the input
// gradient and the weight gradient one after the other, sharing the workspace.
// The weight gradient on the matrix cores (bf16 activations, batches of kHwDwMinB and more):
// workspace = the feature-major bf16 copies of X and dY, then the view's segment lists when the
// descriptor has none.
constexpr int64_t kHwDwMinB = 256;

struct HwDwPlan {
    bool use;
    int64_t Bp, ncb, cw;
    size_t off_x, off_dy, off_tab, total;
};

HwDwPlan plan_hw_dw(int64_t nnz, int64_t O, int64_t I, int64_t B, int dtype, bool colvals, const int32_t *blocks) {
    HwDwPlan p{};
    p.Bp = round_up(B, int64_t(16));
    // the dense products cost O*I*B against the stored products' nnz*B: measured on the matrix cores
    // they win from about 1/12 density (5000 x 5000 at 10 %, B = 4096: 950 against 1235 us; 10k x
    // 10k at 5 %, B = 512: 483 against 302 us)
    const int64_t forced = option(SNACK_OPT_BF16_DW_MFMA);
    const bool dense_enough = forced == 1 || (forced < 0 && 12 * nnz >= O * I);
    p.use = (dtype == SNACK_BF16 || dtype == SNACK_BF16_HW) && B >= kHwDwMinB && nnz > 0 && dense_enough &&
            nnz < (int64_t(1) << 29) && (std::max(O, I) + 320) * p.Bp * 2 < (int64_t(1) << 31);
    if (!p.use) return p;
    const int64_t nkeys = colvals ? I : O, ngather = colvals ? O : I;
    tile_blocks(ngather, p.ncb, p.cw);
    if (nkeys * p.ncb * 4 >= (int64_t(1) << 29)) {
        p.use = false;
        return p;
    }
    size_t at = 0;
    p.off_x = at;
    at = align_up(at + static_cast<size_t>(I * p.Bp) * 2);
    p.off_dy = at;
    at = align_up(at + static_cast<size_t>(O * p.Bp) * 2);
    p.off_tab = at;
    if (!blocks) at = align_up(at + static_cast<size_t>(nkeys * p.ncb) * 16);
    p.total = at;
    return p;
}

struct BwdPlan {
    bool fused;
    int bt, q, nb;  // nb: row bands of the fused kernel (1 or kXcds)
    int64_t bpad;   // batch columns of the feature-major copies (B rounded up to 4)
    size_t off_x, off_dy, off_part, total;
    // split: both gradients tiled, reading X and dY in place; the input gradient's workspace
    // starts at off_spmm, the weight gradient's segment table at off_sddmm.
    // tiled: both gradients in one tiled pass over the column view (tile_bwd_kernel), its segment
    // table and dX partials in the workspace at off_spmm (laid out by sp)
    bool split, tiled;
    SpmmPlan sp;
    SddmmPlan sd;
    size_t off_spmm, off_sddmm;
};

// Smallest lane count per slot of the one-pass backward (1: batches 4, 8, 12 take it too).
constexpr int kFusedMinBt = 1;

// Layers with at least this many entries take the row-banded form of the fused backward pass
// (SNACK_OPT_BAND_MIN_NNZ overrides it).  The backward's form where more than one applies is the
// library's choice unless SNACK_OPT_BWD_FORM names one: 0 the one-pass kernel reading dY rows from
// L2, 1 two tiled passes, 2 one tiled pass.
constexpr int64_t kBandMinNnz = int64_t(1) << 20;

int bwd_form_env() { return static_cast<int>(option(SNACK_OPT_BWD_FORM)); }

int64_t band_min_nnz() {
    const int64_t v = option(SNACK_OPT_BAND_MIN_NNZ);
    return v >= 0 ? v : kBandMinNnz;
}

BwdPlan plan_bwd(int64_t nnz, int64_t O, int64_t I, int64_t B, int dtype, bool aligned16, bool colvals = false) {
    BwdPlan p{};
    const int64_t Bp = pad_batch(B);
    p.bpad = Bp;
    if (nnz > 0 && Bp >= 4 && (std::max(I, O) + 1) * Bp * 4 < (int64_t(1) << 32)) {
        // padded batch Bp = 4*BT*Q: BT lanes per slot (the largest power of two <= 16 that leaves
        // Q <= 4 float4s per lane)
        for (int bt = 16; bt >= kFusedMinBt; bt /= 2) {
            if (Bp % (4 * bt) == 0 && Bp / (4 * bt) <= 4) {
                p.fused = true;
                p.bt = bt;
                p.q = static_cast<int>(Bp / (4 * bt));
                // row bands (one per XCD) once the triple is large enough to spill L2; values in
                // column order are read and written in walk order, and the bands only add waves
                p.nb = !colvals && nnz >= band_min_nnz() ? kXcds : 1;
                break;
            }
        }
    }
    // both gradients tiled (the input gradient over the column view reading the values through
    // col_perm, the weight gradient over the row view), one after the other, instead of the fused
    // pass: values in row order and one 64-column batch tile (with more tiles, or values in column
    // order, the fused pass measured faster)
    // default: values in column order take the one tiled pass (10k x 10k steps, us, against the
    // one-pass kernel reading dY rows from L2: 90 % B = 16 109 / 121, B = 32 127 / 135, 95 %
    // B = 16 68 / 69, B = 32 82 / 81, B = 64 97 / 107); values in row order the two tiled passes
    // (the one tiled pass writes dW through col_perm there, and the scattered stores cost more
    // than the second pass: 95 % B = 64 step 113 against 148 us)
    const int form = bwd_form_env();
    const bool tiled_ok = form == 2 || (form < 0 && colvals);
    if (p.fused && tiled_ok && (Bp == 16 || Bp == 32 || Bp == 64) && Bp * I < (int64_t(1) << 29)) {
        // (the plan of the column-view walk bounds Bp O; X is read in place too)
        const SpmmPlan sp = plan_spmm(nnz, O, I, B, dtype, true, aligned16, colvals);
        if (sp.mapping == kTile && sp.bpad == Bp && sp.tnbt == 1 && !sp.cvals) {
            p.fused = false;
            p.tiled = true;
            p.sp = sp;
            p.off_x = p.off_dy = p.off_spmm = 0;  // X and dY read in place
            p.total = align_up(sp.total);
            return p;
        }
    }
    if (p.fused && form != 0 && form != 2 && !colvals && (Bp == 16 || Bp == 32 || Bp == 64)) {
        const SpmmPlan sp = plan_spmm(nnz, O, I, B, dtype, true, aligned16, colvals);
        const SddmmPlan sd = plan_sddmm(nnz, O, I, B, dtype, colvals);
        if (sp.mapping == kTile && sd.tile && sp.bpad == Bp && sd.bpad == Bp) {
            p.fused = false;
            p.split = true;
            p.sp = sp;
            p.sd = sd;
            size_t at = 0;  // both passes read X and dY in place
            p.off_x = p.off_dy = at;
            p.off_spmm = at;
            at = align_up(at + sp.total);
            p.off_sddmm = at;
            at = align_up(at + 4 * sizeof(int32_t) * static_cast<size_t>(O * sd.tncb));
            p.total = at;
            return p;
        }
    }
    if (p.fused) {
        size_t at = 0;
        p.off_x = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>((I + 1) * Bp));
        p.off_dy = at;
        at = align_up(at + sizeof(float) * static_cast<size_t>((O + 1) * Bp));
        p.off_part = at;
        if (p.nb > 1) at = align_up(at + sizeof(float) * static_cast<size_t>(p.nb * I * Bp));
        p.total = at;
    } else {
        // the separate calls; the weight gradient's segment lists counted as if the descriptor had none
        const HwDwPlan hp = plan_hw_dw(nnz, O, I, B, dtype, colvals, nullptr);
        p.total = std::max(plan_spmm(nnz, O, I, B, dtype, true, aligned16, colvals).total,
                           hp.use ? hp.total : plan_sddmm(nnz, O, I, B, dtype, colvals).total);
    }
    return p;
}

int check_hip(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SNACK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return SNACK_OK;
}

int check_desc(const snack_coo_desc *W, bool need_colview, const char *who) {
    if (!W) return fail(SNACK_ERR_NULL, "%s: descriptor is NULL", who);
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    if (O < 0 || I < 0 || nnz < 0 || O > 2147483647LL || I > 2147483647LL || nnz > 2147483647LL ||
        nnz > O * I)
        return fail(SNACK_ERR_SHAPE, "%s: bad sizes O=%lld I=%lld nnz=%lld", who, (long long)O,
                    (long long)I, (long long)nnz);
    if (nnz > 0 && (!W->rows || !W->cols || !W->vals))
        return fail(SNACK_ERR_NULL, "%s: rows, cols and vals are required", who);
    if (!W->row_offsets) return fail(SNACK_ERR_NULL, "%s: row_offsets is required", who);
    if ((need_colview || W->row_to_col) &&
        (!W->col_offsets || (nnz > 0 && (!W->col_perm || !W->col_rows || !W->col_cols))))
        return fail(SNACK_ERR_NULL, "%s: the column view (col_perm, col_rows, col_cols, col_offsets) is required%s",
                    who, W->row_to_col ? " with values in column order" : "");
    if (W->col_blocks && !W->col_offsets)
        return fail(SNACK_ERR_NULL, "%s: col_blocks needs the column view", who);
    if (reinterpret_cast<uintptr_t>(W->row_blocks) % 16 || reinterpret_cast<uintptr_t>(W->col_blocks) % 16)
        return fail(SNACK_ERR_ALIGN, "%s: row_blocks and col_blocks must be 16-byte aligned", who);
    return SNACK_OK;
}

int check_act(const void *p, int dtype, const char *name, const char *who) {
    if (!p) return fail(SNACK_ERR_NULL, "%s: %s is NULL", who, name);
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a % (dtype == SNACK_F32 ? 4 : 2))
        return fail(SNACK_ERR_ALIGN, "%s: %s is not aligned to its element size", who, name);
    return SNACK_OK;
}

int check_workspace(void *ws, size_t have, size_t need, const char *who) {
    if (need == 0) return SNACK_OK;
    if (!ws || have < need)
        return fail(SNACK_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                    ws ? have : size_t(0));
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(SNACK_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
    return SNACK_OK;
}

// activation [B][F] -> feature-major fp32 [F+1][Bp] in `dst` (row F zero, columns B..Bp-1 zero;
// Bp = 0 means B); with src1 != NULL also [B][F1] -> [F1+1][Bp] in dst1, in the same launch
int launch_to_feature_major(const void *src, int dtype, int64_t B, int64_t F, float *dst, hipStream_t st,
                            const void *src1 = nullptr, int64_t F1 = 0, float *dst1 = nullptr, int64_t Bp = 0) {
    if (Bp < B) Bp = B;
    if (B == 0 || (F == 0 && F1 == 0 && !src1)) return SNACK_OK;
    const int64_t fmax = std::max(F, src1 ? F1 : 0);
    const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, ceil_div(fmax, kTf))),
                    static_cast<unsigned>(ceil_div(Bp, kTb)), src1 ? 2u : 1u);
    // vector loads need rows of F a multiple of 4 (16-byte aligned), vector stores Bp
    const bool vec = Bp % 4 == 0 && F % 4 == 0 && (!src1 || F1 % 4 == 0);
    if (dtype == SNACK_F32) {
        const float *a = static_cast<const float *>(src), *a1 = static_cast<const float *>(src1);
        if (vec) hipLaunchKernelGGL(to_feature_major4_kernel<float>, grid, dim3(kBlock), 0, st, a, dst, F, a1, dst1, F1, B, Bp);
        else hipLaunchKernelGGL(to_feature_major_kernel<float>, grid, dim3(kBlock), 0, st, a, dst, F, a1, dst1, F1, B, Bp);
    } else {
        const bf16_t *a = static_cast<const bf16_t *>(src), *a1 = static_cast<const bf16_t *>(src1);
        if (vec) hipLaunchKernelGGL(to_feature_major4_kernel<bf16_t>, grid, dim3(kBlock), 0, st, a, dst, F, a1, dst1, F1, B, Bp);
        else hipLaunchKernelGGL(to_feature_major_kernel<bf16_t>, grid, dim3(kBlock), 0, st, a, dst, F, a1, dst1, F1, B, Bp);
    }
    return check_hip("to_feature_major");
}

template <typename OutT, int BT>
void launch_segscan_bt(const SpmmPlan &p, int64_t nnz, const int32_t *keys, const int32_t *gidx,
                       const float *vals, const int32_t *perm, const float *opnd, int64_t B,
                       const float *bias, OutT *out, int64_t out_ld, float *head, float *tail,
                       hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(ceil_div(p.nchunks, kWavesPerBlock)),
                    static_cast<unsigned>(ceil_div(B, BT)));
    hipLaunchKernelGGL((segscan_kernel<BT, OutT>), grid, dim3(kBlock), 0, st, nnz, p.chunk, p.nchunks,
                       keys, gidx, vals, perm, opnd, B, bias, out, out_ld, head, tail);
}

template <typename OutT, int BT, int Q>
void launch_rowwave_bt(int64_t nkeys, int64_t nnz, const int32_t *offs, const int32_t *gidx, const float *vals,
                       const int32_t *perm, const float *opnd, int64_t opnd_rows, int64_t B, const float *bias,
                       OutT *out, int64_t out_ld, int64_t nbo, hipStream_t st) {
    const int zero_row = static_cast<int>(opnd_rows);  // the transposed operand's zero row
    // keys with >= 256 entries on average are split over the 4 waves of a workgroup, unless
    // values are read through the column permutation: one wave per key keeps co-resident
    // waves walking rows in step, so those reads share L2 lines
    const bool split = !perm && nnz >= 256 * nkeys;
    const int64_t keys_per_block = split ? 1 : kWavesPerBlock;
    const int64_t blocks = round_up8(ceil_div(nkeys, keys_per_block));
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(ceil_div(B, 4 * BT * Q)));
    if (split)
        hipLaunchKernelGGL((rowwave_kernel<BT, 4, Q, OutT>), grid, dim3(kBlock), 0, st, nkeys, offs, gidx, vals,
                           perm, opnd, zero_row, B, bias, out, out_ld, nbo);
    else
        hipLaunchKernelGGL((rowwave_kernel<BT, 1, Q, OutT>), grid, dim3(kBlock), 0, st, nkeys, offs, gidx, vals,
                           perm, opnd, zero_row, B, bias, out, out_ld, nbo);
}

// out[j] = vals[perm[j]]: the stored values in column-view order
__global__ __launch_bounds__(kBlock) void gather_vals_kernel(const int32_t *__restrict__ perm,
                                                             const float *__restrict__ vals, int64_t n,
                                                             float *__restrict__ out) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (j < n) out[j] = vals[perm[j]];
}

int launch_gather(const int32_t *idx, const float *src, int64_t n, float *dst, hipStream_t st) {
    if (n == 0) return SNACK_OK;
    hipLaunchKernelGGL(gather_vals_kernel, dim3(static_cast<unsigned>(ceil_div(n, kBlock))), dim3(kBlock), 0, st,
                       idx, src, n, dst);
    return check_hip("gather_vals_kernel");
}

template <int VW, int CH, bool VP, typename InT>
int launch_tile_kernel(const SpmmPlan &p, int64_t nkeys, const int32_t *tab, const int32_t *gidx, const float *vals,
                       const int32_t *perm, const InT *act, int64_t opnd_rows, int64_t B, float *part,
                       hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(round_up8(static_cast<int64_t>(p.tncb) * p.tnrb)),
                    static_cast<unsigned>(p.tnbt));
    hipLaunchKernelGGL((tile_spmm_kernel<VW, CH, VP, InT>), grid, dim3(kTileThreads), 0, st,
                       static_cast<int>(nkeys), p.tncb, p.tnrb, p.tcw, p.tkpr, tab, gidx, vals, perm, p.tnnz, act,
                       static_cast<int>(opnd_rows), B, part);
    return check_hip("tile_spmm_kernel");
}

template <int VW, bool VP, typename InT>
int launch_tile_ch(const SpmmPlan &p, int64_t nkeys, const int32_t *tab, const int32_t *gidx, const float *vals,
                   const int32_t *perm, const InT *act, int64_t opnd_rows, int64_t B, float *part, hipStream_t st) {
    // 8 prefetched chunks with permuted values at 64 columns would spill registers; longer
    // segments take their further chunks unprefetched there
    switch (VW == 4 && VP ? std::min(p.tch, 4) : p.tch) {
        case 2: return launch_tile_kernel<VW, 2, VP>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st);
        case 4: return launch_tile_kernel<VW, 4, VP>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st);
        case 8: return launch_tile_kernel<VW, 8, VP>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st);
        default: return fail(SNACK_ERR_INTERNAL, "tile: unsupported chunk count %d", p.tch);
    }
}

template <int VW, typename InT>
int launch_tile_vw(const SpmmPlan &p, int64_t nkeys, const int32_t *tab, const int32_t *gidx, const float *vals,
                   const int32_t *perm, const InT *act, int64_t opnd_rows, int64_t B, float *part, hipStream_t st) {
    if (perm) return launch_tile_ch<VW, true>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st);
    return launch_tile_ch<VW, false>(p, nkeys, tab, gidx, vals, nullptr, act, opnd_rows, B, part, st);
}

// The LDS-tiled gather-reduce: segment table, tiles, block sums (bias, transpose).
int launch_bounds(int64_t nkeys, int ncb, int cw, const int32_t *offs, const int32_t *gidx, int32_t *tab,
                  hipStream_t st) {
    const int64_t waves = ceil_div(nkeys, kSegWindow) * ncb;
    if (waves == 0) return SNACK_OK;
    hipLaunchKernelGGL(tile_segments_kernel, dim3(static_cast<unsigned>(ceil_div(waves, kBlock / kWave))), dim3(kBlock),
                       0, st, static_cast<int>(nkeys), ncb, cw, offs, gidx, reinterpret_cast<int4 *>(tab));
    return check_hip("tile_segments_kernel");
}

// blocks: the layer's segment lists for this walk (snack_coo_desc.row_blocks / col_blocks), or
// NULL to build it in the workspace first.  act: the batch-major operand [B][opnd_rows], in the
// output's type.
template <typename OutT>
int launch_tile(const SpmmPlan &p, int64_t nkeys, const int32_t *offs, const int32_t *gidx, const float *vals,
                const int32_t *perm, const int32_t *blocks, const OutT *act, int64_t opnd_rows, int64_t B,
                const float *bias, OutT *out, char *ws, hipStream_t st) {
    const int32_t *tab = blocks;
    float *part = reinterpret_cast<float *>(ws + p.off_part);
    probe(true, st);
    if (!tab) {
        int32_t *t = reinterpret_cast<int32_t *>(ws + p.off_tab);
        if (int s = launch_bounds(nkeys, p.tncb, p.tcw, offs, gidx, t, st)) return s;
        tab = t;
    }
    int s;
    switch (p.ttb) {
        case 16: s = launch_tile_vw<1>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st); break;
        case 32: s = launch_tile_vw<2>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st); break;
        case 64: s = launch_tile_vw<4>(p, nkeys, tab, gidx, vals, perm, act, opnd_rows, B, part, st); break;
        default: return fail(SNACK_ERR_INTERNAL, "tile: unsupported batch tile %d", p.ttb);
    }
    if (s) return s;
    const unsigned kw = static_cast<unsigned>(4 * kBlock / p.ttb);  // keys per block-sum workgroup
    const dim3 sgrid(static_cast<unsigned>(ceil_div(nkeys, kw)), static_cast<unsigned>(p.tnbt));
    if (p.ttb == 16)
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 16>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(nkeys),
                           p.tncb, B, bias, out, nkeys);
    else if (p.ttb == 32)
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 32>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(nkeys),
                           p.tncb, B, bias, out, nkeys);
    else
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 64>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(nkeys),
                           p.tncb, B, bias, out, nkeys);
    probe(false, st);
    return check_hip("tile_sum_kernel");
}

// The gather-reduce shared by the forward (row order) and the input gradient
// (column view).  nkeys = number of outputs per batch row; offs [nkeys+1].  opnd: the batch-major
// activation (in the output's type) where the plan reads it in place (p.direct), else its fp32
// feature-major copy.
template <typename OutT>
int run_spmm(const SpmmPlan &p, int64_t nkeys, int64_t nnz, const int32_t *keys, const int32_t *offs,
             const int32_t *gidx, const float *vals, const int32_t *perm, const void *opnd_any, int64_t opnd_rows,
             int64_t B, const float *bias, OutT *out, char *ws, hipStream_t st, const int32_t *blocks) {
    if (nkeys == 0 || B == 0) return SNACK_OK;
    const float *opnd = static_cast<const float *>(opnd_any);
    if (p.mapping == kTile) {
        if (p.cvals && perm) {  // several batch tiles: the values gathered into walk order once
            float *cv = reinterpret_cast<float *>(ws + p.off_cvals);
            if (int s = launch_gather(perm, vals, nnz, cv, st)) return s;
            vals = cv;
            perm = nullptr;
        }
        return launch_tile<OutT>(p, nkeys, offs, gidx, vals, perm, blocks, static_cast<const OutT *>(opnd_any),
                                 opnd_rows, B, bias, out, ws, st);
    }
    if (p.mapping == kRowwave) {
        probe(true, st);
        if (p.cvals && perm) {
            float *cv = reinterpret_cast<float *>(ws + p.off_cvals);
            hipLaunchKernelGGL(gather_vals_kernel, dim3(static_cast<unsigned>(ceil_div(nnz, kBlock))), dim3(kBlock), 0,
                               st, perm, vals, nnz, cv);
            vals = cv;
            perm = nullptr;
        }
        switch (p.bt * 8 + p.q) {
#define SNACK_RW(BTV, QV)                                                                                           \
    case BTV * 8 + QV:                                                                                               \
        launch_rowwave_bt<OutT, BTV, QV>(nkeys, nnz, offs, gidx, vals, perm, opnd, opnd_rows, p.bpad, bias, out, nkeys, \
                                         B, st);                                                                    \
        break;
            SNACK_RW(1, 1) SNACK_RW(2, 1) SNACK_RW(4, 1) SNACK_RW(8, 1) SNACK_RW(16, 1)
            SNACK_RW(1, 3) SNACK_RW(2, 3) SNACK_RW(4, 3) SNACK_RW(8, 3) SNACK_RW(16, 3)
            SNACK_RW(16, 4)
#undef SNACK_RW
            default: return fail(SNACK_ERR_INTERNAL, "rowwave: unsupported plan bt=%d q=%d", p.bt, p.q);
        }
        probe(false, st);
        return check_hip("rowwave_kernel");
    }
    float *head = reinterpret_cast<float *>(ws + p.off_head);
    float *tail = reinterpret_cast<float *>(ws + p.off_tail);
    if (p.nchunks > 0) {
        probe(true, st);
        switch (p.bt) {
#define SNACK_SEG(BTV) \
    case BTV: launch_segscan_bt<OutT, BTV>(p, nnz, keys, gidx, vals, perm, opnd, B, bias, out, nkeys, head, tail, st); break;
            SNACK_SEG(1) SNACK_SEG(2) SNACK_SEG(4) SNACK_SEG(8) SNACK_SEG(16) SNACK_SEG(32) SNACK_SEG(64)
#undef SNACK_SEG
            default: return fail(SNACK_ERR_INTERNAL, "segscan: unsupported lane count %d", p.bt);
        }
        probe(false, st);
        if (int s = check_hip("segscan_kernel")) return s;
    }
    const dim3 grid(static_cast<unsigned>(ceil_div(nkeys, kBlock)),
                    static_cast<unsigned>(std::min<int64_t>(B, 65535)));
    hipLaunchKernelGGL(fixup_kernel<OutT>, grid, dim3(kBlock), 0, st, nkeys, B,
                       p.chunk > 0 ? p.chunk : 1, offs, bias, head, tail, out, nkeys);
    return check_hip("fixup_kernel");
}

}  // namespace

namespace {

// Half-precision weights (SNACK_BF16_HW): the MFMA gather-reduce over one view.  K groups: runs
// of the view's blocks split over workgroups so that about kHwWgTarget run (three per CU), their
// partial tiles summed in group order by tile_sum_kernel.  Workspace: the partials (more than
// one group), then the view's segment lists when the descriptor has none.
struct HwPlan {
    int64_t ncb, cw, nkt, nbt, ngy, nkg, bpg;
    bool wide;  // hw_spmm_wide_kernel: batches beyond one tile share each densified slab
    size_t off_part, off_tab, total;
};

HwPlan plan_hw(int64_t nkeys, int64_t ngather, int64_t nnz, int64_t B, const int32_t *blocks) {
    HwPlan p{};
    tile_blocks(ngather, p.ncb, p.cw);
    p.nkt = ceil_div(nkeys, kHwKeys);
    p.nbt = ceil_div(B, kHwTb);
    // keys averaging 64 entries or more: the slab writes cost enough to share them over four
    // batch tiles; with fewer, one batch tile per workgroup keeps more MFMA work in flight
    p.wide = p.nbt > 1 && nnz >= kHwWideMinPerKey * nkeys;
    p.ngy = p.wide ? ceil_div(B, kHwWideTb) : p.nbt;
    // K groups: about kHwWgTarget workgroups (three per CU), or two per CU for the wide kernel
    const int64_t target = p.wide ? 512 : kHwWgTarget;
    const int64_t tiles = std::max<int64_t>(1, p.nkt * p.ngy);
    p.nkg = std::min<int64_t>(p.ncb, std::max<int64_t>(1, ceil_div(target, tiles)));
    p.bpg = ceil_div(p.ncb, p.nkg);
    p.nkg = ceil_div(p.ncb, p.bpg);
    size_t at = 0;
    p.off_part = at;
    if (p.nkg > 1 && nkeys > 0) at = align_up(at + sizeof(float) * static_cast<size_t>(p.nbt * p.nkg * nkeys * kHwTb));
    p.off_tab = at;
    if (!blocks && nkeys > 0) at = align_up(at + static_cast<size_t>(nkeys * p.ncb) * 16);
    p.total = at;
    return p;
}

size_t hw_spmm_bytes(int64_t nkeys, int64_t ngather, int64_t nnz, int64_t B, const int32_t *blocks) {
    if (nkeys == 0 || B == 0) return 0;
    return plan_hw(nkeys, ngather, nnz, B, blocks).total;
}

// What hw_spmm_kernel assumes of a call: 16-byte operand loads from 16-byte aligned rows, 32-bit
// byte offsets into the activations, the entry arrays and the segment lists.
int hw_spmm_check(int64_t nkeys, int64_t ngather, int64_t nnz, int64_t B, const void *act, const char *name,
                  const char *who) {
    if (ngather % 8)
        return fail(SNACK_ERR_SHAPE, "%s: half-precision weights need %s's feature count to be a multiple of 8 (%lld)",
                    who, name, (long long)ngather);
    if (ngather > 0 && reinterpret_cast<uintptr_t>(act) % 16)
        return fail(SNACK_ERR_ALIGN, "%s: half-precision weights need %s 16-byte aligned", who, name);
    if ((B * ngather + 1024) * 2 >= (int64_t(1) << 31))
        return fail(SNACK_ERR_SHAPE, "%s: %s of %lld x %lld elements is beyond the half-precision path's 2^30", who,
                    name, (long long)B, (long long)ngather);
    int64_t ncb, cw;
    tile_blocks(ngather, ncb, cw);
    if (nnz >= (int64_t(1) << 29) || nkeys * ncb * 4 >= (int64_t(1) << 29))
        return fail(SNACK_ERR_SHAPE, "%s: layer beyond the half-precision path's 2^29 entries", who);
    return SNACK_OK;
}

int launch_hw_spmm(int64_t nkeys, int64_t ngather, int64_t nnz, const int32_t *offs, const int32_t *gidx,
                   const float *vals, const int32_t *perm, const int32_t *blocks, const void *act, int64_t B,
                   const float *bias, void *out, char *ws, hipStream_t st) {
    if (nkeys == 0 || B == 0) return SNACK_OK;
    const HwPlan p = plan_hw(nkeys, ngather, nnz, B, blocks);
    const int32_t *tab = blocks;
    if (!tab) {
        int32_t *t = reinterpret_cast<int32_t *>(ws + p.off_tab);
        if (int s = launch_bounds(nkeys, static_cast<int>(p.ncb), static_cast<int>(p.cw), offs, gidx, t, st)) return s;
        tab = t;
    }
    float *part = p.nkg > 1 ? reinterpret_cast<float *>(ws + p.off_part) : nullptr;
    const dim3 grid(static_cast<unsigned>(p.nkt), static_cast<unsigned>(p.ngy), static_cast<unsigned>(p.nkg));
    const int nk = static_cast<int>(nkeys), ng = static_cast<int>(ngather), nc = static_cast<int>(p.ncb),
              w = static_cast<int>(p.cw), bpg = static_cast<int>(p.bpg), nz = static_cast<int>(nnz);
    const bf16_t *a = static_cast<const bf16_t *>(act);
    bf16_t *o = static_cast<bf16_t *>(out);
    probe(true, st);
    if (p.wide && perm)
        hipLaunchKernelGGL((hw_spmm_wide_kernel<true, bf16_t>), grid, dim3(kHwThreads), 0, st, nk, ng, nc, w, bpg,
                           tab, gidx, vals, perm, nz, a, B, bias, o, part);
    else if (p.wide)
        hipLaunchKernelGGL((hw_spmm_wide_kernel<false, bf16_t>), grid, dim3(kHwThreads), 0, st, nk, ng, nc, w, bpg,
                           tab, gidx, vals, nullptr, nz, a, B, bias, o, part);
    else if (perm)
        hipLaunchKernelGGL((hw_spmm_kernel<true, bf16_t>), grid, dim3(kHwThreads), 0, st, nk, ng, nc, w, bpg, tab,
                           gidx, vals, perm, nz, a, B, bias, o, part);
    else
        hipLaunchKernelGGL((hw_spmm_kernel<false, bf16_t>), grid, dim3(kHwThreads), 0, st, nk, ng, nc, w, bpg, tab,
                           gidx, vals, nullptr, nz, a, B, bias, o, part);
    if (int s = check_hip(p.wide ? "hw_spmm_wide_kernel" : "hw_spmm_kernel")) return s;
    if (part) {
        constexpr int kw = 4 * kBlock / kHwTb;
        const dim3 sgrid(static_cast<unsigned>(ceil_div(nkeys, kw)), static_cast<unsigned>(p.nbt));
        hipLaunchKernelGGL((tile_sum_kernel<bf16_t, kHwTb>), sgrid, dim3(kBlock), 0, st, part, nk,
                           static_cast<int>(p.nkg), B, bias, o, nkeys);
        if (int s = check_hip("tile_sum_kernel")) return s;
    }
    probe(false, st);
    return SNACK_OK;
}

// dW over the view the values are stored in (row order, or the column view with values in column
// order), written in that order.
int launch_hw_dw(const HwDwPlan &p, const snack_coo_desc *W, const void *X, const void *dY, int64_t B, float *dW,
                 char *ws, hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    const bool colvals = W->row_to_col != nullptr;
    bf16_t *xt = reinterpret_cast<bf16_t *>(ws + p.off_x), *dyt = reinterpret_cast<bf16_t *>(ws + p.off_dy);
    const dim3 gx(static_cast<unsigned>(ceil_div(I, 64)), static_cast<unsigned>(ceil_div(p.Bp, 64)));
    const dim3 gy(static_cast<unsigned>(ceil_div(O, 64)), static_cast<unsigned>(ceil_div(p.Bp, 64)));
    if (I > 0)
        hipLaunchKernelGGL(bf16_feature_major_kernel, gx, dim3(kBlock), 0, st, static_cast<const bf16_t *>(X), B, I,
                           p.Bp, xt);
    if (O > 0)
        hipLaunchKernelGGL(bf16_feature_major_kernel, gy, dim3(kBlock), 0, st, static_cast<const bf16_t *>(dY), B, O,
                           p.Bp, dyt);
    if (int s = check_hip("bf16_feature_major_kernel")) return s;
    const int64_t nkeys = colvals ? I : O, ngather = colvals ? O : I;
    const int32_t *offs = colvals ? W->col_offsets : W->row_offsets;
    const int32_t *gidx = colvals ? W->col_rows : W->cols;
    const int32_t *tab = colvals ? W->col_blocks : W->row_blocks;
    if (!tab) {
        int32_t *t = reinterpret_cast<int32_t *>(ws + p.off_tab);
        if (int s = launch_bounds(nkeys, static_cast<int>(p.ncb), static_cast<int>(p.cw), offs, gidx, t, st)) return s;
        tab = t;
    }
    const dim3 grid(static_cast<unsigned>(ceil_div(nkeys, kHwDwKeys)), static_cast<unsigned>(3 * p.ncb));
    probe(true, st);
    hipLaunchKernelGGL(hw_sddmm_kernel, grid, dim3(kHwThreads), 0, st, static_cast<int>(nkeys),
                       static_cast<int>(ngather), static_cast<int>(p.ncb), static_cast<int>(p.cw),
                       static_cast<int>(p.Bp), tab, gidx, static_cast<int>(nnz), colvals ? xt : dyt,
                       colvals ? dyt : xt, dW);
    probe(false, st);
    return check_hip("hw_sddmm_kernel");
}
}  // namespace

// ================================================================ C ABI
extern "C" size_t snack_coo_workspace_bytes(int op, const snack_coo_desc *W, int64_t batch, int act_dtype) {
    if (act_dtype != SNACK_F32 && act_dtype != SNACK_BF16 && act_dtype != SNACK_BF16_HW) {
        fail(SNACK_ERR_DTYPE, "workspace_bytes: unknown dtype %d", act_dtype);
        return 0;
    }
    if (check_desc(W, false, "workspace_bytes") || batch < 0) {
        if (batch < 0) fail(SNACK_ERR_SHAPE, "workspace_bytes: negative batch");
        return 0;
    }
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    const bool cv = W->row_to_col != nullptr;
    if (act_dtype == SNACK_BF16_HW) {
        const size_t dx = hw_spmm_bytes(I, O, nnz, batch, W->col_blocks);
        const HwDwPlan hp = plan_hw_dw(nnz, O, I, batch, SNACK_BF16, cv, cv ? W->col_blocks : W->row_blocks);
        const size_t dw = hp.use ? hp.total : plan_sddmm(nnz, O, I, batch, SNACK_BF16, cv).total;
        switch (op) {
            case SNACK_OP_FWD: return hw_spmm_bytes(O, I, nnz, batch, W->row_blocks);
            case SNACK_OP_BWD_INPUT: return dx;
            case SNACK_OP_GRAD_WEIGHT: return dw;
            case SNACK_OP_BWD: return std::max(dx, dw);
            default: fail(SNACK_ERR_DTYPE, "workspace_bytes: unknown op %d", op); return 0;
        }
    }
    switch (op) {
        case SNACK_OP_FWD: return plan_spmm(nnz, I, O, batch, act_dtype, false, false, cv).total;
        case SNACK_OP_BWD_INPUT: return plan_spmm(nnz, O, I, batch, act_dtype, true, vec16(W), cv).total;
        case SNACK_OP_GRAD_WEIGHT: {
            const HwDwPlan hp = plan_hw_dw(nnz, O, I, batch, act_dtype, cv, cv ? W->col_blocks : W->row_blocks);
            return hp.use ? hp.total : plan_sddmm(nnz, O, I, batch, act_dtype, cv).total;
        }
        case SNACK_OP_BWD: return plan_bwd(nnz, O, I, batch, act_dtype, vec16(W), cv).total;
        default: fail(SNACK_ERR_DTYPE, "workspace_bytes: unknown op %d", op); return 0;
    }
}

namespace {

// Batch 1 over a CSR structure (offs [nkeys+1], gidx/vals in walk order, vals through vperm when
// non-NULL): y[key] = bias[key] + sum of vals * x[gidx], then the chunk-edge fix-up.  The forward
// runs it over the row view; with values in column order the input gradient runs it over the
// column view.
int launch_csr1(const SpmmPlan &p, int act_dtype, int64_t nkeys, int64_t nx, int64_t nnz, const int32_t *offs,
                const int32_t *gidx, const float *vals, const int32_t *vperm, const void *x, const float *bias,
                void *y, char *ws, hipStream_t st) {
    float *head = reinterpret_cast<float *>(ws + p.off_head);
    float *tail = reinterpret_cast<float *>(ws + p.off_tail);
    const bool staged = nx <= kStageMaxI;
    const int threads = staged ? kStageThreads : kBlock;
    const dim3 grid(static_cast<unsigned>(round_up8(ceil_div(p.nchunks, threads / kWave))));
    const size_t lds = staged ? sizeof(float) * static_cast<size_t>(nx) : 0;
    const int o = static_cast<int>(nkeys), in = static_cast<int>(nx), nz = static_cast<int>(nnz),
              ch = static_cast<int>(p.chunk), nc = static_cast<int>(p.nchunks);
#define SNACK_CSR1_FWD(T, TH, VP)                                                                                 \
    hipLaunchKernelGGL((csr1_fwd_kernel<T, T, TH, VP>), grid, dim3(TH), lds, st, o, in, nz, ch, nc, offs, gidx, vals, \
                       vperm, static_cast<const T *>(x), bias, static_cast<T *>(y), head, tail)
#define SNACK_CSR1_FWD_T(T)                                   \
    if (staged && vperm) SNACK_CSR1_FWD(T, kStageThreads, true); \
    else if (staged) SNACK_CSR1_FWD(T, kStageThreads, false);    \
    else if (vperm) SNACK_CSR1_FWD(T, kBlock, true);             \
    else SNACK_CSR1_FWD(T, kBlock, false);
    probe(true, st);
    if (act_dtype == SNACK_F32) {
        SNACK_CSR1_FWD_T(float)
    } else {
        SNACK_CSR1_FWD_T(bf16_t)
    }
#undef SNACK_CSR1_FWD_T
#undef SNACK_CSR1_FWD
    probe(false, st);
    if (int s = check_hip("csr1_fwd_kernel")) return s;
    const dim3 fgrid(static_cast<unsigned>(ceil_div(nkeys, kBlock)), 1);
    if (act_dtype == SNACK_F32)
        hipLaunchKernelGGL(fixup_kernel<float>, fgrid, dim3(kBlock), 0, st, nkeys, int64_t(1), p.chunk, offs, bias,
                           head, tail, static_cast<float *>(y), nkeys);
    else
        hipLaunchKernelGGL(fixup_kernel<bf16_t>, fgrid, dim3(kBlock), 0, st, nkeys, int64_t(1), p.chunk, offs, bias,
                           head, tail, static_cast<bf16_t *>(y), nkeys);
    return check_hip("fixup_kernel");
}

}  // namespace

extern "C" int snack_coo_fwd(const snack_coo_desc *W, const void *X, int64_t batch, int act_dtype,
                             const float *bias, void *Y, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
    try {
        const char *who = "snack_coo_fwd";
        if (int s = check_desc(W, false, who)) return s;
        if (act_dtype != SNACK_F32 && act_dtype != SNACK_BF16 && act_dtype != SNACK_BF16_HW)
            return fail(SNACK_ERR_DTYPE, "%s: unknown dtype %d", who, act_dtype);
        if (batch < 0 || batch > kMaxBatch)
            return fail(SNACK_ERR_SHAPE, "%s: batch %lld outside [0, 2^21]", who, (long long)batch);
        const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
        if (batch == 0 || O == 0) return snack::ok();
        if (I > 0) { if (int s = check_act(X, act_dtype, "X", who)) return s; }
        if (int s = check_act(Y, act_dtype, "Y", who)) return s;
        if (act_dtype == SNACK_BF16_HW) {
            if (int s = hw_spmm_check(O, I, nnz, batch, X, "X", who)) return s;
            if (int s = check_workspace(workspace, workspace_bytes, hw_spmm_bytes(O, I, nnz, batch, W->row_blocks), who)) return s;
            // the row walk reads values in column order through row_to_col
            if (int s = launch_hw_spmm(O, I, nnz, W->row_offsets, W->cols, W->vals, W->row_to_col, W->row_blocks, X,
                                       batch, bias, Y, static_cast<char *>(workspace), static_cast<hipStream_t>(hip_stream)))
                return s;
            return snack::ok();
        }
        const SpmmPlan p = plan_spmm(nnz, I, O, batch, act_dtype, false, false, W->row_to_col != nullptr);
        if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        char *ws = static_cast<char *>(workspace);
        // the row walk reads values in column order through row_to_col
        const float *vals = W->vals;
        const int32_t *vperm = W->row_to_col;
        if (p.mapping == kCsr1) {
            if (int s = launch_csr1(p, act_dtype, O, I, nnz, W->row_offsets, W->cols, vals, vperm, X, bias, Y, ws, st))
                return s;
            return snack::ok();
        }
        const void *xt = X;
        if (!p.direct) {
            float *dst = reinterpret_cast<float *>(ws + p.off_opnd);
            if (int s = launch_to_feature_major(X, act_dtype, batch, I, dst, st, nullptr, 0, nullptr, p.bpad)) return s;
            xt = dst;
        }
        int s;
        if (act_dtype == SNACK_F32)
            s = run_spmm<float>(p, O, nnz, W->rows, W->row_offsets, W->cols, vals, vperm, xt, I, batch, bias,
                                static_cast<float *>(Y), ws, st, W->row_blocks);
        else
            s = run_spmm<bf16_t>(p, O, nnz, W->rows, W->row_offsets, W->cols, vals, vperm, xt, I, batch, bias,
                                 static_cast<bf16_t *>(Y), ws, st, W->row_blocks);
        return s ? s : snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_fwd: unexpected exception");
    }
}

// Workspace of snack_coo_fwd_noalloc: every device the library runs on holds its own copy.  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[SNACK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up on its first use on that device.
int scratch_address(void **out, const char *who) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return check_hip(who);
    if (dev < 0 || dev >= kScratchDevices)
        return fail(SNACK_ERR_INTERNAL, "%s: device %d beyond the %d the scratch table holds", who, dev,
                    kScratchDevices);
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(SNACK_ERR_HIP, "%s: address of the static scratch on device %d: %s", who, dev,
                            hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SNACK_OK;
}
}  // namespace

extern "C" int snack_coo_fwd_noalloc(const snack_coo_desc *W, const void *X, int64_t batch, int act_dtype,
                                     const float *bias, void *Y, void *hip_stream) {
    try {
        const char *who = "snack_coo_fwd_noalloc";
        const size_t need = snack_coo_workspace_bytes(SNACK_OP_FWD, W, batch, act_dtype);
        // need == 0: no workspace, or invalid arguments, which snack_coo_fwd reports
        if (need == 0) return snack_coo_fwd(W, X, batch, act_dtype, bias, Y, nullptr, 0, hip_stream);
        if (need > SNACK_NOALLOC_SCRATCH_BYTES)
            return fail(SNACK_ERR_WORKSPACE, "%s: this call needs %zu bytes of workspace, more than the %zu of the static scratch",
                        who, need, static_cast<size_t>(SNACK_NOALLOC_SCRATCH_BYTES));
        void *ws = nullptr;
        if (int s = scratch_address(&ws, who)) return s;
        return snack_coo_fwd(W, X, batch, act_dtype, bias, Y, ws, SNACK_NOALLOC_SCRATCH_BYTES, hip_stream);
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_fwd_noalloc: unexpected exception");
    }
}

extern "C" int snack_coo_bwd_input(const snack_coo_desc *W, const void *dY, int64_t batch, int act_dtype,
                                   void *dX, float *db, void *workspace, size_t workspace_bytes,
                                   void *hip_stream) {
    try {
        const char *who = "snack_coo_bwd_input";
        if (int s = check_desc(W, true, who)) return s;
        if (act_dtype != SNACK_F32 && act_dtype != SNACK_BF16 && act_dtype != SNACK_BF16_HW)
            return fail(SNACK_ERR_DTYPE, "%s: unknown dtype %d", who, act_dtype);
        if (batch < 0 || batch > kMaxBatch)
            return fail(SNACK_ERR_SHAPE, "%s: batch %lld outside [0, 2^21]", who, (long long)batch);
        const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        if (batch > 0 && O > 0) { if (int s = check_act(dY, act_dtype, "dY", who)) return s; }
        if (batch > 0 && I > 0) { if (int s = check_act(dX, act_dtype, "dX", who)) return s; }
        if (act_dtype == SNACK_BF16_HW && batch > 0 && I > 0) {
            if (int s = hw_spmm_check(I, O, nnz, batch, dY, "dY", who)) return s;
        }
        if (db && O > 0) {
            if (reinterpret_cast<uintptr_t>(db) % 4) return fail(SNACK_ERR_ALIGN, "%s: db misaligned", who);
            const dim3 grid(static_cast<unsigned>(ceil_div(O, kBlock)));
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(bias_grad_kernel<float>, grid, dim3(kBlock), 0, st, O, batch,
                                   static_cast<const float *>(dY), db);
            else
                hipLaunchKernelGGL(bias_grad_kernel<bf16_t>, grid, dim3(kBlock), 0, st, O, batch,
                                   static_cast<const bf16_t *>(dY), db);
            if (int s = check_hip("bias_grad_kernel")) return s;
        }
        if (batch == 0 || I == 0) return snack::ok();
        const bool colvals = W->row_to_col != nullptr;
        if (act_dtype == SNACK_BF16_HW) {
            if (int s = check_workspace(workspace, workspace_bytes, hw_spmm_bytes(I, O, nnz, batch, W->col_blocks), who)) return s;
            // the column walk reads values in row order through col_perm, values in column order in place
            if (int s = launch_hw_spmm(I, O, nnz, W->col_offsets, W->col_rows, W->vals, colvals ? nullptr : W->col_perm,
                                       W->col_blocks, dY, batch, nullptr, dX, static_cast<char *>(workspace), st))
                return s;
            return snack::ok();
        }
        const SpmmPlan p = plan_spmm(nnz, O, I, batch, act_dtype, true, vec16(W), colvals);
        if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
        char *ws = static_cast<char *>(workspace);
        // batch 1 walks the column view as the forward walks the rows (values in row order through
        // col_perm)
        if (p.mapping == kCsr1) {
            if (int s = launch_csr1(p, act_dtype, I, O, nnz, W->col_offsets, W->col_rows, W->vals,
                                    colvals ? nullptr : W->col_perm, dY, nullptr, dX, ws, st))
                return s;
            return snack::ok();
        }
        const float *rvals = W->vals;  // the row walks below run with values in row order only
        if (p.mapping == kCsr1Priv) {
            float *partial = reinterpret_cast<float *>(ws + p.off_head);
            const size_t lds = sizeof(float) * static_cast<size_t>(kPrivWaves * I);
            static std::atomic<uint64_t> lds_f32{0}, lds_bf16{0};  // up to 160 KB of LDS
            const size_t lds_max = sizeof(float) * kPrivWaves * kPrivMaxI;
            if (int s = act_dtype == SNACK_F32
                            ? allow_lds(reinterpret_cast<const void *>(&csr1_dxpriv_kernel<float>), lds_max, lds_f32,
                                        "csr1_dxpriv_kernel")
                            : allow_lds(reinterpret_cast<const void *>(&csr1_dxpriv_kernel<bf16_t>), lds_max,
                                        lds_bf16, "csr1_dxpriv_kernel"))
                return s;
            const int o = static_cast<int>(O), in = static_cast<int>(I), nz = static_cast<int>(nnz),
                      ch = static_cast<int>(p.chunk), nc = static_cast<int>(p.nchunks);
            const dim3 grid(static_cast<unsigned>(p.nparts));
            probe(true, st);
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(csr1_dxpriv_kernel<float>, grid, dim3(kPrivWaves * kWave), lds, st, o, in, nz, ch,
                                   nc, W->row_offsets, W->cols, rvals, static_cast<const float *>(dY), partial);
            else
                hipLaunchKernelGGL(csr1_dxpriv_kernel<bf16_t>, grid, dim3(kPrivWaves * kWave), lds, st, o, in, nz, ch,
                                   nc, W->row_offsets, W->cols, rvals, static_cast<const bf16_t *>(dY), partial);
            probe(false, st);
            if (int s = check_hip("csr1_dxpriv_kernel")) return s;
            const dim3 rgrid(static_cast<unsigned>(ceil_div(I, kWave)));
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(dx_reduce_kernel<float>, rgrid, dim3(kReduceThreads), 0, st, I, p.nparts, partial,
                                   static_cast<float *>(dX));
            else
                hipLaunchKernelGGL(dx_reduce_kernel<bf16_t>, rgrid, dim3(kReduceThreads), 0, st, I, p.nparts, partial,
                                   static_cast<bf16_t *>(dX));
            if (int s = check_hip("dx_reduce_kernel")) return s;
            return snack::ok();
        }
        if (p.mapping == kScatter) {
            float *partial = reinterpret_cast<float *>(ws + p.off_head);
            const size_t lds = sizeof(float) * static_cast<size_t>(batch * I);
            probe(true, st);
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(dx_scatter_kernel<float>, dim3(static_cast<unsigned>(p.nchunks)),
                                   dim3(kScatterThreads), lds, st, nnz, p.chunk, O, I, batch, W->rows, W->cols,
                                   rvals, static_cast<const float *>(dY), partial);
            else
                hipLaunchKernelGGL(dx_scatter_kernel<bf16_t>, dim3(static_cast<unsigned>(p.nchunks)),
                                   dim3(kScatterThreads), lds, st, nnz, p.chunk, O, I, batch, W->rows, W->cols,
                                   rvals, static_cast<const bf16_t *>(dY), partial);
            probe(false, st);
            if (int s = check_hip("dx_scatter_kernel")) return s;
            const int64_t n = batch * I;
            const dim3 grid(static_cast<unsigned>(ceil_div(n, kWave)));
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(dx_reduce_kernel<float>, grid, dim3(kReduceThreads), 0, st, n, p.nchunks, partial,
                                   static_cast<float *>(dX));
            else
                hipLaunchKernelGGL(dx_reduce_kernel<bf16_t>, grid, dim3(kReduceThreads), 0, st, n, p.nchunks, partial,
                                   static_cast<bf16_t *>(dX));
            if (int s = check_hip("dx_reduce_kernel")) return s;
            return snack::ok();
        }
        const void *dyt = dY;
        if (!p.direct) {
            float *dst = reinterpret_cast<float *>(ws + p.off_opnd);
            if (int s = launch_to_feature_major(dY, act_dtype, batch, O, dst, st, nullptr, 0, nullptr, p.bpad))
                return s;
            dyt = dst;
        }
        // the column walk reads values in row order through col_perm, values in column order in place
        const int32_t *vperm = colvals ? nullptr : W->col_perm;
        int s;
        if (act_dtype == SNACK_F32)
            s = run_spmm<float>(p, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, vperm, dyt, O,
                                batch, nullptr, static_cast<float *>(dX), ws, st, W->col_blocks);
        else
            s = run_spmm<bf16_t>(p, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, vperm, dyt, O,
                                 batch, nullptr, static_cast<bf16_t *>(dX), ws, st, W->col_blocks);
        return s ? s : snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_bwd_input: unexpected exception");
    }
}

extern "C" int snack_coo_grad_weight(const snack_coo_desc *W, const void *X, const void *dY, int64_t batch,
                                     int act_dtype, float *dW_out, void *workspace, size_t workspace_bytes,
                                     void *hip_stream) {
    try {
        const char *who = "snack_coo_grad_weight";
        if (int s = check_desc(W, false, who)) return s;
        if (act_dtype != SNACK_F32 && act_dtype != SNACK_BF16 && act_dtype != SNACK_BF16_HW)
            return fail(SNACK_ERR_DTYPE, "%s: unknown dtype %d", who, act_dtype);
        if (act_dtype == SNACK_BF16_HW) act_dtype = SNACK_BF16;  // dW does not read the weights
        if (batch < 0 || batch > kMaxBatch)
            return fail(SNACK_ERR_SHAPE, "%s: batch %lld outside [0, 2^21]", who, (long long)batch);
        const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
        if (nnz == 0) return snack::ok();
        if (!dW_out) return fail(SNACK_ERR_NULL, "%s: dW is NULL", who);
        if (reinterpret_cast<uintptr_t>(dW_out) % 4) return fail(SNACK_ERR_ALIGN, "%s: dW misaligned", who);
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        if (batch == 0) {
            hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(ceil_div(nnz, kBlock))), dim3(kBlock), 0,
                               st, dW_out, nnz);
            if (int s = check_hip("zero_kernel")) return s;
            return snack::ok();
        }
        if (int s = check_act(X, act_dtype, "X", who)) return s;
        if (int s = check_act(dY, act_dtype, "dY", who)) return s;
        const bool colvals = W->row_to_col != nullptr;
        const HwDwPlan hp = plan_hw_dw(nnz, O, I, batch, act_dtype, colvals, colvals ? W->col_blocks : W->row_blocks);
        if (hp.use) {
            if (int s = check_workspace(workspace, workspace_bytes, hp.total, who)) return s;
            if (int s = launch_hw_dw(hp, W, X, dY, batch, dW_out, static_cast<char *>(workspace), st)) return s;
            return snack::ok();
        }
        const SddmmPlan p = plan_sddmm(nnz, O, I, batch, act_dtype, colvals);
        if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
        char *ws = static_cast<char *>(workspace);
        // the kernels write dW in row order; with values in column order into the workspace, and
        // finish() gathers it into column order through col_perm
        float *dW = colvals ? reinterpret_cast<float *>(ws + p.off_dw) : dW_out;
        auto finish = [&]() -> int {
            if (colvals) {
                if (int s = launch_gather(W->col_perm, dW, nnz, dW_out, st)) return s;
            }
            return snack::ok();
        };
        if (p.csr1) {
            // dW[k] = dY[row] * X[col] along the row view, or (values in column order) along the
            // column view with the roles of X and dY swapped, straight into column order
            const int64_t nk = colvals ? I : O, nx = colvals ? O : I;
            const int32_t *woffs = colvals ? W->col_offsets : W->row_offsets;
            const int32_t *widx = colvals ? W->col_rows : W->cols;
            const void *wx = colvals ? dY : X, *wdy = colvals ? X : dY;
            float *wdw = colvals ? dW_out : dW;
            const bool staged = nx <= kStageMaxI;
            const int threads = staged ? kStageThreads : kBlock;
            const dim3 grid(static_cast<unsigned>(round_up8(ceil_div(p.waves, threads / kWave))));
            const size_t lds = staged ? sizeof(float) * static_cast<size_t>(nx) : 0;
            const int o = static_cast<int>(nk), in = static_cast<int>(nx), nz = static_cast<int>(nnz),
                      ch = static_cast<int>(p.steps), nc = static_cast<int>(p.waves);
#define SNACK_CSR1_DW(T, TH)                                                                                  \
    hipLaunchKernelGGL((csr1_dw_kernel<T, TH>), grid, dim3(TH), lds, st, o, in, nz, ch, nc, woffs, widx,            \
                       static_cast<const T *>(wx), static_cast<const T *>(wdy), wdw)
            probe(true, st);
            if (act_dtype == SNACK_F32) {
                if (staged) SNACK_CSR1_DW(float, kStageThreads);
                else SNACK_CSR1_DW(float, kBlock);
            } else {
                if (staged) SNACK_CSR1_DW(bf16_t, kStageThreads);
                else SNACK_CSR1_DW(bf16_t, kBlock);
            }
#undef SNACK_CSR1_DW
            probe(false, st);
            if (int s = check_hip("csr1_dw_kernel")) return s;
            return snack::ok();
        }
        if (p.tile) {
            if (int s = launch_tile_sddmm(p, W, X, dY, batch, act_dtype, dW,
                                          reinterpret_cast<int32_t *>(ws + p.off_tab), st))
                return s;
            return finish();
        }
        const float *xt = static_cast<const float *>(X);
        const float *dyt = static_cast<const float *>(dY);
        if (!p.x_direct) {
            float *dst = reinterpret_cast<float *>(ws + p.off_x);
            if (int s = launch_to_feature_major(X, act_dtype, batch, I, dst, st, nullptr, 0, nullptr, p.bpad)) return s;
            xt = dst;
        }
        if (!p.dy_direct) {
            float *dst = reinterpret_cast<float *>(ws + p.off_dy);
            if (int s = launch_to_feature_major(dY, act_dtype, batch, O, dst, st, nullptr, 0, nullptr, p.bpad))
                return s;
            dyt = dst;
        }
        const int64_t blocks = round_up8(ceil_div(p.waves, kWavesPerBlock));
        const dim3 grid(static_cast<unsigned>(blocks));
        probe(true, st);
        if (p.rowq > 0) {
            // rows averaging >= 256 entries are split over the 4 waves of a workgroup
            const bool split = nnz >= 256 * O;
            const dim3 rgrid(static_cast<unsigned>(round_up8(ceil_div(O, split ? 1 : kWavesPerBlock))));
            const int zero_row = static_cast<int>(I);
#define SNACK_ROWSD(BTV, WPRV, QV)                                                                           \
    hipLaunchKernelGGL((rowsddmm_kernel<BTV, WPRV, QV, 8, false>), rgrid, dim3(kBlock), 0, st, O, W->row_offsets, \
                       W->cols, xt, zero_row, dyt, p.bpad, dW)
#define SNACK_ROWSD_Q(BTV, WPRV)                         \
    do {                                                 \
        if (p.rowq == 1) SNACK_ROWSD(BTV, WPRV, 1);      \
        else if (p.rowq == 2) SNACK_ROWSD(BTV, WPRV, 2); \
        else if (p.rowq == 3) SNACK_ROWSD(BTV, WPRV, 3); \
        else SNACK_ROWSD(BTV, WPRV, 4);                  \
    } while (0)
#define SNACK_ROWSD_BT(BTV)                 \
    if (split) SNACK_ROWSD_Q(BTV, 4);       \
    else SNACK_ROWSD_Q(BTV, 1);
            if (p.slices > 1) {
                // slice k: columns [256k, 256k + 256) of the copies (one launch per slice, in order)
                for (int64_t k = 0; k < p.slices; ++k) {
#define SNACK_ROWSD_SLICE(WPRV, ACCV)                                                                          \
    hipLaunchKernelGGL((rowsddmm_kernel<16, WPRV, 4, 2, ACCV>), rgrid, dim3(kBlock), 0, st, O, W->row_offsets, W->cols, \
                       xt + 256 * k, zero_row, dyt + 256 * k, p.bpad, dW)
                    if (split) {
                        if (k > 0) SNACK_ROWSD_SLICE(4, true);
                        else SNACK_ROWSD_SLICE(4, false);
                    } else {
                        if (k > 0) SNACK_ROWSD_SLICE(1, true);
                        else SNACK_ROWSD_SLICE(1, false);
                    }
#undef SNACK_ROWSD_SLICE
                }
            } else if (p.bt == 16) {
                SNACK_ROWSD_BT(16)
            } else if (p.bt == 8) {
                SNACK_ROWSD_BT(8)
            } else if (p.bt == 4) {
                SNACK_ROWSD_BT(4)
            } else if (p.bt == 2) {
                SNACK_ROWSD_BT(2)
            } else {
                SNACK_ROWSD_BT(1)
            }
#undef SNACK_ROWSD_BT
#undef SNACK_ROWSD_Q
#undef SNACK_ROWSD
        } else if (p.wide) {
            const int64_t q = batch / (4 * p.bt);  // float4s per lane (exact when it is cached)
            const bool exact = batch % (4 * p.bt) == 0;
#define SNACK_WIDE(BTV, QV)                                                                            \
    hipLaunchKernelGGL((sddmm_wide_kernel<BTV, QV>), grid, dim3(kBlock), 0, st, nnz, p.per_wave, W->rows, \
                       W->cols, xt, dyt, batch, dW)
            if (exact && q == 1 && p.bt == 16) SNACK_WIDE(16, 1);
            else if (exact && q == 2 && p.bt == 16) SNACK_WIDE(16, 2);
            else if (exact && q == 1 && p.bt == 8) SNACK_WIDE(8, 1);
            else if (exact && q == 1 && p.bt == 4) SNACK_WIDE(4, 1);
            else if (p.bt == 16) SNACK_WIDE(16, 0);
            else if (p.bt == 8) SNACK_WIDE(8, 0);
            else SNACK_WIDE(4, 0);
#undef SNACK_WIDE
        } else switch (p.bt * 8 + p.vw) {
#define SNACK_SDDMM(BTV, VWV)                                                                          \
    case BTV * 8 + VWV:                                                                                \
        hipLaunchKernelGGL((sddmm_kernel<BTV, VWV>), grid, dim3(kBlock), 0, st, nnz, p.steps, W->rows, \
                           W->cols, xt, dyt, batch, dW);                                               \
        break;
            SNACK_SDDMM(1, 1) SNACK_SDDMM(2, 1) SNACK_SDDMM(4, 1) SNACK_SDDMM(8, 1) SNACK_SDDMM(16, 1)
            SNACK_SDDMM(1, 4) SNACK_SDDMM(2, 4) SNACK_SDDMM(4, 4) SNACK_SDDMM(8, 4) SNACK_SDDMM(16, 4)
#undef SNACK_SDDMM
            default: return fail(SNACK_ERR_INTERNAL, "%s: unsupported plan bt=%d vw=%d", who, p.bt, p.vw);
        }
        probe(false, st);
        if (int s = check_hip("sddmm_kernel")) return s;
        return finish();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_grad_weight: unexpected exception");
    }
}

namespace {

template <typename OutT, int BT, int NB, bool COLV>
void launch_colbwd_q(int q, dim3 grid, hipStream_t st, int64_t I, const snack_coo_desc *W, const float *xt,
                     const float *dyt, int zero_row, int64_t B, OutT *dX, float *dW, float *part, int64_t nbo) {
    const int nnz = static_cast<int>(W->nnz);
#define SNACK_COLBWD(QV)                                                                                            \
    hipLaunchKernelGGL((colbwd_kernel<BT, QV, NB, OutT, COLV>), grid, dim3(kBlock), 0, st, I, W->col_offsets,     \
                       W->col_rows, W->col_perm, W->vals, xt, dyt, zero_row, B, dX, dW, W->row_offsets, nnz, part, \
                       nbo)
    if (q == 1) SNACK_COLBWD(1);
    else if (q == 2) SNACK_COLBWD(2);
    else if (q == 3) SNACK_COLBWD(3);
    else SNACK_COLBWD(4);
#undef SNACK_COLBWD
}

template <typename OutT, int NB, bool COLV = false>
void launch_colbwd_nb(const BwdPlan &p, dim3 grid, hipStream_t st, int64_t I, const snack_coo_desc *W,
                      const float *xt, const float *dyt, int zero_row, int64_t B, OutT *dX, float *dW, float *part) {
    const int64_t Bp = p.bpad;  // the copies' batch columns; B of them are real
    if (p.bt == 16)
        launch_colbwd_q<OutT, 16, NB, COLV>(p.q, grid, st, I, W, xt, dyt, zero_row, Bp, dX, dW, part, B);
    else if (p.bt == 8)
        launch_colbwd_q<OutT, 8, NB, COLV>(p.q, grid, st, I, W, xt, dyt, zero_row, Bp, dX, dW, part, B);
    else if (p.bt == 4)
        launch_colbwd_q<OutT, 4, NB, COLV>(p.q, grid, st, I, W, xt, dyt, zero_row, Bp, dX, dW, part, B);
    else if (p.bt == 2)
        launch_colbwd_q<OutT, 2, NB, COLV>(p.q, grid, st, I, W, xt, dyt, zero_row, Bp, dX, dW, part, B);
    else
        launch_colbwd_q<OutT, 1, NB, COLV>(p.q, grid, st, I, W, xt, dyt, zero_row, Bp, dX, dW, part, B);
}

template <typename OutT>
int launch_colbwd(const BwdPlan &p, hipStream_t st, int64_t I, const snack_coo_desc *W, const float *xt,
                  const float *dyt, int zero_row, int64_t B, OutT *dX, float *dW, float *part) {
    if (p.nb == 1) {
        // one wave per column, 4 consecutive columns per workgroup, each XCD an eighth of the columns;
        // values in column order are read and dW written at the walk's own positions
        const dim3 grid(static_cast<unsigned>(round_up8(ceil_div(I, kWavesPerBlock))));
        if (W->row_to_col)
            launch_colbwd_nb<OutT, 1, true>(p, grid, st, I, W, xt, dyt, zero_row, B, dX, dW, part);
        else
            launch_colbwd_nb<OutT, 1>(p, grid, st, I, W, xt, dyt, zero_row, B, dX, dW, part);
        return check_hip("colbwd_kernel");
    }
    const dim3 grid(static_cast<unsigned>(kXcds * ceil_div(I, kWavesPerBlock)));
    launch_colbwd_nb<OutT, kXcds>(p, grid, st, I, W, xt, dyt, zero_row, B, dX, dW, part);
    if (int s = check_hip("colbwd_kernel")) return s;
    const dim3 sgrid(static_cast<unsigned>(ceil_div(I, kTf)), static_cast<unsigned>(ceil_div(B, kTb)));
    hipLaunchKernelGGL((band_sum_kernel<kXcds, OutT>), sgrid, dim3(kBlock), 0, st, part, I, p.bpad, B, dX);
    return check_hip("band_sum_kernel");
}

}  // namespace

// Both gradients tiled (BwdPlan.split): db, the input gradient over the column view (values
// through col_perm), the weight gradient over the row view; the tiles read X and dY in place.
// The timing probe brackets both gradients' kernels.
static int run_split_bwd(const BwdPlan &p, const snack_coo_desc *W, const void *X, const void *dY, int64_t batch,
                  int act_dtype, void *dX, float *db, float *dW, char *ws, hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    if (db) {
        const dim3 grid(static_cast<unsigned>(ceil_div(O, kBlock)));
        if (act_dtype == SNACK_F32)
            hipLaunchKernelGGL(bias_grad_kernel<float>, grid, dim3(kBlock), 0, st, O, batch,
                               static_cast<const float *>(dY), db);
        else
            hipLaunchKernelGGL(bias_grad_kernel<bf16_t>, grid, dim3(kBlock), 0, st, O, batch,
                               static_cast<const bf16_t *>(dY), db);
        if (int s = check_hip("bias_grad_kernel")) return s;
    }
    probe(true, st);
    ++g_probe_mute;
    int s = act_dtype == SNACK_F32
                ? run_spmm<float>(p.sp, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, W->col_perm, dY,
                                  O, batch, nullptr, static_cast<float *>(dX), ws + p.off_spmm, st, W->col_blocks)
                : run_spmm<bf16_t>(p.sp, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, W->col_perm,
                                   dY, O, batch, nullptr, static_cast<bf16_t *>(dX), ws + p.off_spmm, st,
                                   W->col_blocks);
    if (!s)
        s = launch_tile_sddmm(p.sd, W, X, dY, batch, act_dtype, dW, reinterpret_cast<int32_t *>(ws + p.off_sddmm),
                              st);
    --g_probe_mute;
    if (s) return s;
    probe(false, st);
    return snack::ok();
}

template <int VW, int CH, bool VP, typename InT>
int launch_tile_bwd_kernel(const SpmmPlan &sp, int64_t I, int64_t O, int64_t B, const int32_t *tab,
                           const snack_coo_desc *W, const InT *dY, const InT *X, float *part, float *dW,
                           hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(round_up8(static_cast<int64_t>(sp.tncb) * sp.tnrb)));
    hipLaunchKernelGGL((tile_bwd_kernel<VW, CH, VP, InT>), grid, dim3(kTileThreads), 0, st, static_cast<int>(I),
                       sp.tncb, sp.tnrb, sp.tcw, sp.tkpr, tab, W->col_rows, W->vals, VP ? W->col_perm : nullptr,
                       sp.tnnz, dY, static_cast<int>(O), X, B, part, dW);
    return check_hip("tile_bwd_kernel");
}

template <int VW, bool VP, typename InT>
int launch_tile_bwd_ch(const SpmmPlan &sp, int64_t I, int64_t O, int64_t B, const int32_t *tab,
                       const snack_coo_desc *W, const InT *dY, const InT *X, float *part, float *dW, hipStream_t st) {
    if (sp.tch <= 2) return launch_tile_bwd_kernel<VW, 2, VP>(sp, I, O, B, tab, W, dY, X, part, dW, st);
    return launch_tile_bwd_kernel<VW, 4, VP>(sp, I, O, B, tab, W, dY, X, part, dW, st);
}

// Both gradients in one tiled pass (BwdPlan.tiled): db, tile_bwd_kernel over the column view
// reading X and dY in place (dW written directly; values in row order read and dW written through
// col_perm), then the block sums of dX.  The probe brackets the last two.
template <typename OutT>
int run_tiled_bwd(const BwdPlan &p, const snack_coo_desc *W, const OutT *X, const OutT *dY, int64_t batch,
                  OutT *dX, float *db, float *dW, char *ws, hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features;
    const SpmmPlan &sp = p.sp;
    if (db) {
        const dim3 grid(static_cast<unsigned>(ceil_div(O, kBlock)));
        hipLaunchKernelGGL(bias_grad_kernel<OutT>, grid, dim3(kBlock), 0, st, O, batch, dY, db);
        if (int s = check_hip("bias_grad_kernel")) return s;
    }
    char *sws = ws + p.off_spmm;
    float *part = reinterpret_cast<float *>(sws + sp.off_part);
    probe(true, st);
    const int32_t *tab = W->col_blocks;
    if (!tab) {
        int32_t *t = reinterpret_cast<int32_t *>(sws + sp.off_tab);
        if (int s = launch_bounds(I, sp.tncb, sp.tcw, W->col_offsets, W->col_rows, t, st)) return s;
        tab = t;
    }
    const bool vp = W->row_to_col == nullptr;  // values in row order: read and write through col_perm
    int s;
    switch (sp.ttb * 2 + (vp ? 1 : 0)) {
        case 33: s = launch_tile_bwd_ch<1, true>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        case 32: s = launch_tile_bwd_ch<1, false>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        case 65: s = launch_tile_bwd_ch<2, true>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        case 64: s = launch_tile_bwd_ch<2, false>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        case 129: s = launch_tile_bwd_ch<4, true>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        case 128: s = launch_tile_bwd_ch<4, false>(sp, I, O, batch, tab, W, dY, X, part, dW, st); break;
        default: return fail(SNACK_ERR_INTERNAL, "tiled backward: unsupported batch tile %d", sp.ttb);
    }
    if (s) return s;
    const unsigned kw = static_cast<unsigned>(4 * kBlock / sp.ttb);
    const dim3 sgrid(static_cast<unsigned>(ceil_div(I, kw)), 1);
    if (sp.ttb == 16)
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 16>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(I), sp.tncb,
                           batch, nullptr, dX, I);
    else if (sp.ttb == 32)
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 32>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(I), sp.tncb,
                           batch, nullptr, dX, I);
    else
        hipLaunchKernelGGL((tile_sum_kernel<OutT, 64>), sgrid, dim3(kBlock), 0, st, part, static_cast<int>(I), sp.tncb,
                           batch, nullptr, dX, I);
    probe(false, st);
    return check_hip("tile_sum_kernel");
}

extern "C" int snack_coo_bwd_is_fused(const snack_coo_desc *W, int64_t batch, int act_dtype) {
    try {
        if (int s = check_desc(W, true, "snack_coo_bwd_is_fused")) return -s;
        if (act_dtype == SNACK_BF16_HW) return 0;
        const BwdPlan p = plan_bwd(W->nnz, W->out_features, W->in_features, batch, act_dtype, vec16(W),
                                   W->row_to_col != nullptr);
        return p.fused || p.tiled ? 1 : 0;
    } catch (...) {
        return -fail(SNACK_ERR_INTERNAL, "snack_coo_bwd_is_fused: unexpected exception");
    }
}

extern "C" int snack_coo_bwd(const snack_coo_desc *W, const void *X, const void *dY, int64_t batch, int act_dtype,
                             void *dX, float *db, float *dW, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
    try {
        const char *who = "snack_coo_bwd";
        if (int s = check_desc(W, true, who)) return s;
        if (act_dtype != SNACK_F32 && act_dtype != SNACK_BF16 && act_dtype != SNACK_BF16_HW)
            return fail(SNACK_ERR_DTYPE, "%s: unknown dtype %d", who, act_dtype);
        if (batch < 0 || batch > kMaxBatch)
            return fail(SNACK_ERR_SHAPE, "%s: batch %lld outside [0, 2^21]", who, (long long)batch);
        if (act_dtype == SNACK_BF16_HW) {
            // the input gradient on MFMA, then the weight gradient (which does not read the weights)
            if (int s = snack_coo_bwd_input(W, dY, batch, act_dtype, dX, db, workspace, workspace_bytes, hip_stream))
                return s;
            return snack_coo_grad_weight(W, X, dY, batch, act_dtype, dW, workspace, workspace_bytes, hip_stream);
        }
        const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
        const BwdPlan p = plan_bwd(nnz, O, I, batch, act_dtype, vec16(W), W->row_to_col != nullptr);
        if (p.tiled) {
            if (int s = check_act(X, act_dtype, "X", who)) return s;
            if (int s = check_act(dY, act_dtype, "dY", who)) return s;
            if (int s = check_act(dX, act_dtype, "dX", who)) return s;
            if (!dW) return fail(SNACK_ERR_NULL, "%s: dW is NULL", who);
            if (reinterpret_cast<uintptr_t>(dW) % 4) return fail(SNACK_ERR_ALIGN, "%s: dW misaligned", who);
            if (db && reinterpret_cast<uintptr_t>(db) % 4) return fail(SNACK_ERR_ALIGN, "%s: db misaligned", who);
            if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
            char *ws = static_cast<char *>(workspace);
            hipStream_t st = static_cast<hipStream_t>(hip_stream);
            const int s = act_dtype == SNACK_F32
                              ? run_tiled_bwd<float>(p, W, static_cast<const float *>(X),
                                                     static_cast<const float *>(dY), batch, static_cast<float *>(dX),
                                                     db, dW, ws, st)
                              : run_tiled_bwd<bf16_t>(p, W, static_cast<const bf16_t *>(X),
                                                      static_cast<const bf16_t *>(dY), batch,
                                                      static_cast<bf16_t *>(dX), db, dW, ws, st);
            return s ? s : snack::ok();
        }
        if (p.split) {
            if (int s = check_act(X, act_dtype, "X", who)) return s;
            if (int s = check_act(dY, act_dtype, "dY", who)) return s;
            if (int s = check_act(dX, act_dtype, "dX", who)) return s;
            if (!dW) return fail(SNACK_ERR_NULL, "%s: dW is NULL", who);
            if (reinterpret_cast<uintptr_t>(dW) % 4) return fail(SNACK_ERR_ALIGN, "%s: dW misaligned", who);
            if (db && reinterpret_cast<uintptr_t>(db) % 4) return fail(SNACK_ERR_ALIGN, "%s: db misaligned", who);
            if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
            return run_split_bwd(p, W, X, dY, batch, act_dtype, dX, db, dW, static_cast<char *>(workspace),
                                 static_cast<hipStream_t>(hip_stream));
        }
        if (!p.fused) {
            if (int s = snack_coo_bwd_input(W, dY, batch, act_dtype, dX, db, workspace, workspace_bytes, hip_stream))
                return s;
            return snack_coo_grad_weight(W, X, dY, batch, act_dtype, dW, workspace, workspace_bytes, hip_stream);
        }
        if (int s = check_act(X, act_dtype, "X", who)) return s;
        if (int s = check_act(dY, act_dtype, "dY", who)) return s;
        if (int s = check_act(dX, act_dtype, "dX", who)) return s;
        if (!dW) return fail(SNACK_ERR_NULL, "%s: dW is NULL", who);
        if (reinterpret_cast<uintptr_t>(dW) % 4) return fail(SNACK_ERR_ALIGN, "%s: dW misaligned", who);
        if (db && reinterpret_cast<uintptr_t>(db) % 4) return fail(SNACK_ERR_ALIGN, "%s: db misaligned", who);
        if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
        hipStream_t st = static_cast<hipStream_t>(hip_stream);
        char *ws = static_cast<char *>(workspace);
        if (db) {
            const dim3 grid(static_cast<unsigned>(ceil_div(O, kBlock)));
            if (act_dtype == SNACK_F32)
                hipLaunchKernelGGL(bias_grad_kernel<float>, grid, dim3(kBlock), 0, st, O, batch,
                                   static_cast<const float *>(dY), db);
            else
                hipLaunchKernelGGL(bias_grad_kernel<bf16_t>, grid, dim3(kBlock), 0, st, O, batch,
                                   static_cast<const bf16_t *>(dY), db);
            if (int s = check_hip("bias_grad_kernel")) return s;
        }
        float *xt = reinterpret_cast<float *>(ws + p.off_x);
        float *dyt = reinterpret_cast<float *>(ws + p.off_dy);
        if (int s = launch_to_feature_major(X, act_dtype, batch, I, xt, st, dY, O, dyt, p.bpad)) return s;
        // one wave per column: co-resident waves then walk their columns' rows in step, so the
        // vals reads and dW writes through the column permutation share L2 lines (splitting
        // long columns over 4 waves scatters them over the whole triple at once)
        const int zero_row = static_cast<int>(O);
        float *part = reinterpret_cast<float *>(ws + p.off_part);
        probe(true, st);
        int s = act_dtype == SNACK_F32
                    ? launch_colbwd<float>(p, st, I, W, xt, dyt, zero_row, batch, static_cast<float *>(dX), dW, part)
                    : launch_colbwd<bf16_t>(p, st, I, W, xt, dyt, zero_row, batch, static_cast<bf16_t *>(dX), dW,
                                            part);
        probe(false, st);
        if (s) return s;
        return snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_bwd: unexpected exception");
    }
}

extern "C" int snack_coo_set_probe(void *start_event, void *stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr))
        return fail(SNACK_ERR_NULL, "snack_coo_set_probe: give both events or neither");
    g_probe_start = static_cast<hipEvent_t>(start_event);
    g_probe_stop = static_cast<hipEvent_t>(stop_event);
    return snack::ok();
}

namespace {
__global__ __launch_bounds__(kBlock) void invert_perm_kernel(const int32_t *__restrict__ perm, int64_t n,
                                                             int32_t *__restrict__ inv) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (j < n) inv[perm[j]] = static_cast<int32_t>(j);
}
}  // namespace

extern "C" int64_t snack_coo_block_offsets_count(const snack_coo_desc *W, int view) {
    if (!W) {
        fail(SNACK_ERR_NULL, "snack_coo_block_offsets_count: descriptor is NULL");
        return -1;
    }
    if (view != SNACK_VIEW_ROWS && view != SNACK_VIEW_COLS) {
        fail(SNACK_ERR_DTYPE, "snack_coo_block_offsets_count: unknown view %d", view);
        return -1;
    }
    const int64_t keys = view == SNACK_VIEW_ROWS ? W->out_features : W->in_features;
    int64_t ncb, cw;
    tile_blocks(view == SNACK_VIEW_ROWS ? W->in_features : W->out_features, ncb, cw);
    return keys * ncb * 4;
}

extern "C" int snack_coo_block_offsets(const snack_coo_desc *W, int view, int32_t *out, void *hip_stream) {
    try {
        const char *who = "snack_coo_block_offsets";
        if (view != SNACK_VIEW_ROWS && view != SNACK_VIEW_COLS)
            return fail(SNACK_ERR_DTYPE, "%s: unknown view %d", who, view);
        if (int s = check_desc(W, view == SNACK_VIEW_COLS, who)) return s;
        const bool rows = view == SNACK_VIEW_ROWS;
        const int64_t keys = rows ? W->out_features : W->in_features;
        if (keys == 0) return snack::ok();
        if (!out) return fail(SNACK_ERR_NULL, "%s: out is NULL", who);
        if (reinterpret_cast<uintptr_t>(out) % 16) return fail(SNACK_ERR_ALIGN, "%s: out must be 16-byte aligned", who);
        int64_t ncb, cw;
        tile_blocks(rows ? W->in_features : W->out_features, ncb, cw);
        if (keys * ncb * 4 >= (int64_t(1) << 31)) return fail(SNACK_ERR_SHAPE, "%s: table too large", who);
        if (int s = launch_bounds(keys, static_cast<int>(ncb), static_cast<int>(cw), rows ? W->row_offsets : W->col_offsets,
                                  rows ? W->cols : W->col_rows, out, static_cast<hipStream_t>(hip_stream)))
            return s;
        return snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_block_offsets: unexpected exception");
    }
}

extern "C" int snack_coo_invert_perm(const int32_t *perm, int64_t n, int32_t *inv, void *hip_stream) {
    try {
        if (n < 0 || n > 2147483647LL) return fail(SNACK_ERR_SHAPE, "snack_coo_invert_perm: bad length %lld", (long long)n);
        if (n == 0) return snack::ok();
        if (!perm || !inv) return fail(SNACK_ERR_NULL, "snack_coo_invert_perm: perm and inv are required");
        if (reinterpret_cast<uintptr_t>(perm) % 4 || reinterpret_cast<uintptr_t>(inv) % 4)
            return fail(SNACK_ERR_ALIGN, "snack_coo_invert_perm: misaligned array");
        hipLaunchKernelGGL(invert_perm_kernel, dim3(static_cast<unsigned>(ceil_div(n, kBlock))), dim3(kBlock), 0,
                           static_cast<hipStream_t>(hip_stream), perm, n, inv);
        if (int s = check_hip("invert_perm_kernel")) return s;
        return snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_invert_perm: unexpected exception");
    }
}

extern "C" int snack_coo_gather_f32(const float *src, const int32_t *idx, int64_t n, float *dst, void *hip_stream) {
    try {
        if (n < 0 || n > 2147483647LL) return fail(SNACK_ERR_SHAPE, "snack_coo_gather_f32: bad length %lld", (long long)n);
        if (n == 0) return snack::ok();
        if (!src || !idx || !dst) return fail(SNACK_ERR_NULL, "snack_coo_gather_f32: src, idx and dst are required");
        if (reinterpret_cast<uintptr_t>(src) % 4 || reinterpret_cast<uintptr_t>(idx) % 4 ||
            reinterpret_cast<uintptr_t>(dst) % 4)
            return fail(SNACK_ERR_ALIGN, "snack_coo_gather_f32: misaligned array");
        if (int s = launch_gather(idx, src, n, dst, static_cast<hipStream_t>(hip_stream))) return s;
        return snack::ok();
    } catch (...) {
        return fail(SNACK_ERR_INTERNAL, "snack_coo_gather_f32: unexpected exception");
    }
}
