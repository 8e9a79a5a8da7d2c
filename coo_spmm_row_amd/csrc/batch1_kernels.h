// batch1_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Batch-1 and small-batch input-gradient and CSR-stream kernels (K6, K7, K8, K9).
#pragma once

namespace {

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

}  // namespace
