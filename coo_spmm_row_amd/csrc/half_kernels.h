// half_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Half-precision path on the bf16 matrix cores (K15, K16).
#pragma once

namespace {

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

}  // namespace
