// rowmap_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Untiled gather-reduce mappings over the sorted triple: the segmented scan over
// chunks of entries with its fix-up (K2) and one wave per key with float4 gathers (K1).
#pragma once

namespace {

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
// For batches that are multiples of 4.  A workgroup of 16 waves owns 16/WPR
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
// key through LDS.  The workgroup's keys are consecutive; their results are
// staged in LDS and written with consecutive threads on consecutive keys of one batch row, so each
// row of the batch-major output gets one run of 16 / WPR keys per workgroup instead of one
// scattered 2- or 4-byte store per key (written per key, those stores cost about as much as the
// rest of the kernel at batch 1024).  The operand including its zero row is below 4 GB.  B is the
// operand's batch columns (a multiple of 4; zero columns pad a batch of nbo columns), nbo the
// columns stored.
constexpr int kRwThreads = 1024;
constexpr int kRwWaves = kRwThreads / kWave;

template <int BT, int WPR, int Q, typename OutT>
__global__ __launch_bounds__(kRwThreads) void rowwave_kernel(
    int64_t nkeys, const int32_t *__restrict__ offs, const int32_t *__restrict__ gidx,
    const float *__restrict__ vals, const int32_t *__restrict__ perm, const float *__restrict__ opnd, int zero_row,
    int64_t B, const float *__restrict__ bias, OutT *__restrict__ out, int64_t out_ld, int64_t nbo) {
    constexpr int S = kWave / BT;
    constexpr int UQ = 8 / Q;
    constexpr int U = (S * UQ <= kWave) ? UQ : kWave / S;  // S*U divides 64
    constexpr int KPB = kRwWaves / WPR;                   // keys per workgroup
    constexpr int TBC = 4 * BT * Q;                       // batch columns of the tile
    constexpr int OLD = TBC + 4;                          // floats per staged output row
    __shared__ float4 part[WPR > 1 ? kRwWaves : 1][Q][BT];
    __shared__ __align__(16) float ost[KPB][OLD];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int e = lane / BT, t = lane % BT;
    const int64_t k0 = xcd_block() * KPB;
    const int64_t r = k0 + wave / WPR;
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
        float *row = ost[wave / WPR];
#pragma unroll
        for (int q = 0; q < Q; ++q)
            *reinterpret_cast<float4 *>(row + 4 * t + 4 * q * BT) =
                make_float4(acc[q].x + bv, acc[q].y + bv, acc[q].z + bv, acc[q].w + bv);
    }
    __syncthreads();
    // columns past the batch (never staged) and keys past the layer are not written
    const int64_t c0 = static_cast<int64_t>(blockIdx.y) * TBC;
    for (int i = threadIdx.x; i < KPB * TBC; i += kRwThreads) {
        const int k = i % KPB, c = i / KPB;
        if (k0 + k < nkeys && c0 + c < nbo) store_act(out, (c0 + c) * out_ld + k0 + k, ost[k][c]);
    }
}

}  // namespace
