// snack_coo.hip -- libsnack_coo for MI355X (gfx950, CDNA4, wave64): the host-side planners and
// launchers and the C ABI; the kernels are in the headers included below, one per family.
//
// The SNACK layer keeps its weight W (O x I) as a COO triple sorted by (row, col) and runs three
// sparse products on it:
//   forward      Y[b,o]  = bias[o] + sum_{k: rows[k]=o} vals[k] X[b,cols[k]]   (Algorithm 1)
//   input grad   dX[b,i] = sum_{k: cols[k]=i} vals[k] dY[b,rows[k]]            (Section 3.4)
//   weight grad  dW[k]   = sum_b dY[b,rows[k]] X[b,cols[k]]                     (Section 3.4)
// The paper's CUDA mapping (Section 3.2: one thread per non-zero and batch column, atomics into
// C) is not used.  The forward and the input gradient are the same gather-reduce over a sorted
// view: the forward over the row order, the input gradient over the column view (W^T with the
// indices swapped, as Section 3.4 states).  Every output element is produced by one lane or by a
// fixed-order sum of partials, so results are deterministic and no float atomics are used.
//
//   dev_common.h      launch constants, bf16 element I/O, DPP sums and reduce-scatters, the
//                     XCD-aware workgroup order
//   layout_kernels.h  batch-major to feature-major copies for the untiled gathers, clears, db
//   rowmap_kernels.h  untiled gather-reduce: segmented scan over chunks of entries with its
//                     fix-up (balanced by nnz: power-law rows are fine), one wave per key
//   tile_kernels.h    LDS-tiled walks for large layers: a 1024-thread workgroup stages a block
//                     of about 625 operand rows of one batch tile (up to 160 KB) read in place
//                     from the batch-major activations and walks its keys' segments there;
//                     forward and input gradient write per-block partials that tile_sum_kernel
//                     adds in block order; the weight gradient and the one-pass backward (both
//                     gradients from one staged dY block)
//   half_kernels.h    the opt-in half-precision path: bf16 weights and activations on the bf16
//                     matrix cores over tiles of W made dense in LDS, and the bf16 weight
//                     gradient as dense products sampled at the stored entries
//   sddmm_kernels.h   untiled weight gradients and the fused column backward
//   batch1_kernels.h  batch-1 and small-batch kernels: CSR streams over the rows or the column
//                     view, private LDS copies of dX
// The planners below choose one of them per call from the layer's shape, the batch and the
// activation type; the choice never depends on the values.

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

#include "dev_common.h"
#include "layout_kernels.h"
#include "rowmap_kernels.h"
#include "tile_kernels.h"
#include "half_kernels.h"
#include "sddmm_kernels.h"
#include "batch1_kernels.h"

namespace {

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
        // wider batches in multiples of 256: slices of 256 columns in one launch (each gathers
        // its part of the X rows once per entry; the per-entry kernel re-reads the whole dY row
        // per entry).  Against the per-entry kernel: GPT-2 3072->768 weight gradient at batch 512
        // 11.8 against 19.5 us, 5000 x 5000 at 99 % at batch 1024 97 against 115 us.
        if (p.rowq == 0 && Bp % 256 == 0) {
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
    // shared: the input gradient over the column view and the weight gradient both by the
    // row-wave kernels, which read feature-major copies of dY (and X): one copy of each made once,
    // in the weight gradient's workspace at off_sddmm (laid out by sd); the input gradient's
    // workspace at off_spmm
    bool split, tiled, shared;
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
        const SpmmPlan sp = plan_spmm(nnz, O, I, B, dtype, true, aligned16, colvals);
        const SddmmPlan sd = plan_sddmm(nnz, O, I, B, dtype, colvals);
        p.total = std::max(sp.total, hp.use ? hp.total : sd.total);
        // both by the row-wave kernels on copies of the same padding: the copies made once
        // (GPT-2 768->3072 at batch 1024: the step's second 12.6 MB copy of dY and its launch)
        if (nnz > 0 && B > 0 && I > 0 && O > 0 && !hp.use && sp.mapping == kRowwave && !sp.direct &&
            sd.rowq > 0 && !sd.csr1 && !sd.tile && !sd.x_direct && !sd.dy_direct && sp.bpad == sd.bpad) {
            p.shared = true;
            p.sp = sp;
            p.sd = sd;
            p.off_sddmm = 0;
            p.off_spmm = align_up(sd.total);
            p.total = align_up(p.off_spmm + sp.total);
        }
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
    const int64_t keys_per_block = split ? kRwWaves / 4 : kRwWaves;
    const int64_t blocks = round_up8(ceil_div(nkeys, keys_per_block));
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(ceil_div(B, 4 * BT * Q)));
    if (split)
        hipLaunchKernelGGL((rowwave_kernel<BT, 4, Q, OutT>), grid, dim3(kRwThreads), 0, st, nkeys, offs, gidx, vals,
                           perm, opnd, zero_row, B, bias, out, out_ld, nbo);
    else
        hipLaunchKernelGGL((rowwave_kernel<BT, 1, Q, OutT>), grid, dim3(kRwThreads), 0, st, nkeys, offs, gidx, vals,
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

namespace {

// The row-wise weight gradient (rowsddmm_kernel, SddmmPlan.rowq > 0) over the feature-major
// copies xt [I+1][bpad] and dyt [O+1][bpad], written to dW in row order.
int launch_rowsddmm(const SddmmPlan &p, const snack_coo_desc *W, const float *xt, const float *dyt, float *dW,
                    hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    // rows averaging >= 256 entries are split over the 4 waves of a workgroup
    const bool split = nnz >= 256 * O;
    const dim3 rgrid(static_cast<unsigned>(round_up8(ceil_div(O, split ? 1 : kWavesPerBlock))));
    const int zero_row = static_cast<int>(I);
#define SNACK_ROWSD(BTV, WPRV, QV)                                                                           \
    hipLaunchKernelGGL((rowsddmm_kernel<BTV, WPRV, QV, 8>), rgrid, dim3(kBlock), 0, st, O, W->row_offsets, \
               W->cols, xt, zero_row, dyt, p.bpad, 1, dW)
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
        // slices of 256 columns of the copies, added in order inside one launch
        const int ns = static_cast<int>(p.slices);
        if (split)
            hipLaunchKernelGGL((rowsddmm_kernel<16, 4, 4, 2>), rgrid, dim3(kBlock), 0, st, O, W->row_offsets,
                               W->cols, xt, zero_row, dyt, p.bpad, ns, dW);
        else
            hipLaunchKernelGGL((rowsddmm_kernel<16, 1, 4, 2>), rgrid, dim3(kBlock), 0, st, O, W->row_offsets,
                               W->cols, xt, zero_row, dyt, p.bpad, ns, dW);
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
    return check_hip("rowsddmm_kernel");
}

}  // namespace

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
            if (int s = launch_rowsddmm(p, W, xt, dyt, dW, st)) return s;
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

// Both gradients by the row-wave kernels (BwdPlan.shared): db; X and dY copied feature-major
// once (one launch for both); the input gradient over the column view reading the dY copy; the
// weight gradient over the row view reading both copies (in row order, then through col_perm when
// the values are in column order).  The timing probe brackets both gradients' kernels.
static int run_shared_bwd(const BwdPlan &p, const snack_coo_desc *W, const void *X, const void *dY, int64_t batch,
                          int act_dtype, void *dX, float *db, float *dW, char *ws, hipStream_t st) {
    const int64_t O = W->out_features, I = W->in_features, nnz = W->nnz;
    const bool colvals = W->row_to_col != nullptr;
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
    char *wsd = ws + p.off_sddmm;
    float *xt = reinterpret_cast<float *>(wsd + p.sd.off_x);
    float *dyt = reinterpret_cast<float *>(wsd + p.sd.off_dy);
    if (int s = launch_to_feature_major(X, act_dtype, batch, I, xt, st, dY, O, dyt, p.sd.bpad)) return s;
    probe(true, st);
    ++g_probe_mute;
    const int32_t *vperm = colvals ? nullptr : W->col_perm;
    int s = act_dtype == SNACK_F32
                ? run_spmm<float>(p.sp, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, vperm, dyt, O,
                                  batch, nullptr, static_cast<float *>(dX), ws + p.off_spmm, st, W->col_blocks)
                : run_spmm<bf16_t>(p.sp, I, nnz, W->col_cols, W->col_offsets, W->col_rows, W->vals, vperm, dyt, O,
                                   batch, nullptr, static_cast<bf16_t *>(dX), ws + p.off_spmm, st, W->col_blocks);
    float *dwr = colvals ? reinterpret_cast<float *>(wsd + p.sd.off_dw) : dW;
    if (!s) s = launch_rowsddmm(p.sd, W, xt, dyt, dwr, st);
    --g_probe_mute;
    if (s) return s;
    probe(false, st);
    if (colvals) {
        if (int e = launch_gather(W->col_perm, dwr, nnz, dW, st)) return e;
    }
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
        if (p.shared) {
            if (int s = check_act(X, act_dtype, "X", who)) return s;
            if (int s = check_act(dY, act_dtype, "dY", who)) return s;
            if (int s = check_act(dX, act_dtype, "dX", who)) return s;
            if (!dW) return fail(SNACK_ERR_NULL, "%s: dW is NULL", who);
            if (reinterpret_cast<uintptr_t>(dW) % 4) return fail(SNACK_ERR_ALIGN, "%s: dW misaligned", who);
            if (db && reinterpret_cast<uintptr_t>(db) % 4) return fail(SNACK_ERR_ALIGN, "%s: db misaligned", who);
            if (int s = check_workspace(workspace, workspace_bytes, p.total, who)) return s;
            return run_shared_bwd(p, W, X, dY, batch, act_dtype, dX, db, dW, static_cast<char *>(workspace),
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
