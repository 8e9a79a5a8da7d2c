// sddmm_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Untiled weight-gradient kernels and the fused column backward (K3, K3b, K4, K5).
#pragma once

namespace {

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
// t+BT, .. of the feature-major dY row, Q of them), takes the row's entries 64
// at a time with their X rows as 32-bit float4 offsets (the next 64 prefetched;
// lanes past the row's end point at X's zero row), gathers U entries per slot
// in flight and reduce-scatters each slot's U dot products over its BT lanes by DPP.
// ld: row stride (floats) of the feature-major copies.  A batch wider than 4*BT*Q is taken in
// nslices slices of 4*BT*Q columns within each chunk of 64 entries: the slice's dY registers are
// loaded once per chunk, and each step's partial dot products are added in slice order in
// registers (NSTEP of them per lane), so dW is written once.  UQ: entries per slot in flight (at
// most 64/S); the sliced form measured fastest with 2, a single slice with 8.
template <int BT, int WPR, int Q, int UQ>
__global__ __launch_bounds__(kBlock) void rowsddmm_kernel(int64_t O, const int32_t *__restrict__ offs,
                                                          const int32_t *__restrict__ cols,
                                                          const float *__restrict__ xt, int zero_row,
                                                          const float *__restrict__ dyt, int64_t ld, int nslices,
                                                          float *__restrict__ dW) {
    constexpr int S = kWave / BT;
    constexpr int U = (S * UQ <= kWave) ? UQ : kWave / S;  // S*U divides 64
    constexpr int KPB = kWavesPerBlock / WPR;
    constexpr int TBC = 4 * BT * Q;                        // batch columns per slice
    constexpr int NSTEP = kWave / (S * U);                 // steps per chunk of 64 entries
    // the slot's U dot products are reduce-scattered over its BT lanes: lane t with t % R == 0
    // ends with entry h + e + S*(t / R) of step h, and the wave's stores are contiguous
    constexpr int R = BT / U;
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
    auto load_dy = [&](int k) {
#pragma unroll
        for (int q = 0; q < Q; ++q) dyv[q] = y4[k * (TBC / 4) + q * BT];
    };
    if (nslices == 1) load_dy(0);
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
        float acc[NSTEP];
#pragma unroll
        for (int j = 0; j < NSTEP; ++j) acc[j] = 0.f;
        for (int k = 0; k < nslices; ++k) {
            if (nslices > 1) load_dy(k);
            const uint32_t xs = 16u * static_cast<uint32_t>(k * (TBC / 4));  // slice k's byte offset
#pragma unroll
            for (int j = 0; j < NSTEP; ++j) {
                const int h = j * S * U;
                if (h < n) {
                    const int sa = (h + e) << 2;
                    float4 x[U][Q];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t o =
                            16u * static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sa + 4 * S * u, co)) + xs;
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
                    acc[j] = k == 0 ? dsum : acc[j] + dsum;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NSTEP; ++j) {
            const int src = j * S * U + (t / R) * S + e;
            if (t % R == 0 && src < n) dW[base + src] = acc[j];
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

}  // namespace
