// tile_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// LDS-tiled walks (K12, K13, K14): the segment lists, the gather-reduce, the sampled
// product and the one-pass backward over a block of staged operand rows, and the block sum.
#pragma once

namespace {

// ---------------------------------------------------------------- LDS-tiled gather-reduce
// The same gather-reduce as rowwave (out[key][:] = sum over the key's entries of
// vals * opnd[gidx][:]), with the operand rows served from LDS instead of L2.  W is cut into
// tiles of (a range of keys) x (a block of cw operand rows); a 1024-thread workgroup stages its
// block of the operand, read in place from the batch-major activations (cw rows of 64 batch
// columns, 256 B each, plus one zero row: up to 160 KB, gfx950's LDS) once, then walks its keys'
// segments inside the block.  The
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
// of 16 lanes holds entries j = 0..15 of its slot's chunk), one group ahead of the compute (two
// when the values are read through a permutation, the values themselves one ahead).
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
            const float r = chunk_reduce_scatter(p, m - 16 * c, j);
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
        const float r = chunk_reduce_scatter(p, nst, j);
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

}  // namespace
