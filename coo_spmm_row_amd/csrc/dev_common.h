// dev_common.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Device-side helpers every kernel family uses: launch constants, bf16 element
// I/O, DPP cross-lane sums and reduce-scatters, the XCD-aware workgroup order.
#pragma once

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

// Reduce-scatter over a row of 16 lanes of the first U = 4 or 8 of 16 values, each landing on
// the low lanes: lane t returns the row's sum of v[t mod U] (for a chunk of 16 sampled products
// of which only the first U were computed).  The halving stages pair lanes by mirror within 8
// (bit 2, for U = 8), xor 2 and xor 1, keeping the half the lane's own bit selects, so lane t
// keeps index t mod U; the rest are plain sums over rotations of the row by 4 (for U = 4) and by
// 8, which pair lanes with the same low bits, hence the same kept index: 11 instructions for
// U = 4 and 22 for U = 8, against 45 for the full reduce-scatter.
template <int U>
__device__ __forceinline__ float row_reduce_scatter_low(const float (&v)[16], int t) {
    static_assert(U == 4 || U == 8, "4 or 8 values");
    float w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) w[j] = v[j];
    if constexpr (U == 8) reduce_scatter_stage<0x141, 2, 8, U>(w, t);
    reduce_scatter_stage<0x4E, 1, 4, U>(w, t);
    reduce_scatter_stage<0xB1, 0, 2, U>(w, t);
    if constexpr (U == 4) w[0] += dpp_move<0x124>(w[0]);  // row_ror:4
    w[0] += dpp_move<0x128>(w[0]);                         // row_ror:8
    return w[0];
}

// The reduce-scatter of a chunk of 16 sampled products over a row of 16 lanes, of which the
// first nst (uniform across the wave) were computed and the rest are zero: lane t < nst returns
// the row's sum of v[t].
__device__ __forceinline__ float chunk_reduce_scatter(const float (&v)[16], int nst, int t) {
    if (nst <= 4) return row_reduce_scatter_low<4>(v, t);
    if (nst <= 8) return row_reduce_scatter_low<8>(v, t);
    return group_reduce_scatter<16, 16>(v, t);
}

// Logical workgroup index such that each XCD (blockIdx.x % 8 under round-robin
// dispatch) works on one contiguous eighth of the logical range.  gridDim.x is
// a multiple of 8; callers drop logical ids beyond their real count.
__device__ __forceinline__ int64_t xcd_block() {
    const int64_t per = gridDim.x / kXcds;
    return (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

}  // namespace
