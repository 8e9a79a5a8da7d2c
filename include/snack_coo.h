/*
 * snack_coo.h -- C ABI of the SNACK truly-sparse linear layer on MI355X (gfx950).
 *
 * Source: "Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural Networks
 * on GPU" (Badour, van Keulen, Mocanu; arXiv:2610.04093).
 *
 * The layer's weight W (out_features x in_features, O x I) exists only as its
 * stored entries, a COO triple (rows[k], cols[k], vals[k]) for k < nnz
 * (Section 3.1 and Figure 1; the triple is defined in Appendix B, Table 7).
 * Three device operations make up the layer's hot path:
 *
 *   forward      Y  = X W^T + b        Y[b,o]  = bias[o] + sum_{k: rows[k]=o} vals[k] X[b,cols[k]]
 *   input grad   dX = dY W             dX[b,i] = sum_{k: cols[k]=i} vals[k] dY[b,rows[k]]
 *   weight grad  dW[k] = sum_b dY[b,rows[k]] X[b,cols[k]]   (only on the stored entries)
 *
 * (Algorithm 1 for the forward product; Section 3.4 and Appendix F,
 * "Full gradient derivation", for both gradients.)  Two host operations sit
 * beside them: the row-sorted COO builder (Table 7's COO, CSR index pointer
 * and CSC view) and the magnitude prune-and-regrow topology update of
 * Appendix G, which regrows with the uniform initializer of Algorithm 2.
 *
 * Conventions for every function below:
 *  - Return value: SNACK_OK (0) or a positive snack_status; no exception
 *    crosses the ABI.  snack_last_error() gives a message for the last
 *    failure on the calling thread.
 *  - Ownership: the caller allocates and frees every buffer.  The library
 *    keeps no state between calls (apart from the optional per-thread timing
 *    probe of snack_coo_set_probe) and never allocates device memory; device
 *    scratch comes from the caller's workspace (see snack_coo_workspace_bytes).
 *  - Sizes: O, I and nnz fit in int32; batch is at most 2^21.
 *  - Streams: device calls only enqueue work on hip_stream (a hipStream_t;
 *    NULL = the default stream) and never synchronise.  Device faults surface
 *    at the caller's next synchronisation.  Calls on different streams that
 *    share a workspace race.
 *  - Layout: activations are row-major and batch-major (X[batch][I],
 *    Y[batch][O], dY[batch][O], dX[batch][I]), contiguous.  Indices are int32,
 *    0-based; vals, bias, dW and db are fp32.  Activations are fp32 or bf16
 *    (SNACK_BF16: X, dY read as bf16; Y, dX written as bf16 rounded to nearest
 *    even from fp32 accumulators).  SNACK_BF16_HW, the half-precision path
 *    (the Tensor-Core SNACK-COO for fp16/bf16 that the SNACK paper names as
 *    future work, Conclusion, Limitations, and Future Work): activations as for
 *    SNACK_BF16, and the weights in bf16 too -- each stored fp32 value is
 *    rounded to bf16 (nearest even) as it is read -- with the products of the
 *    forward and the input gradient run on gfx950's bf16 matrix cores (MFMA)
 *    over tiles of W made dense in LDS (never in device memory); fp32
 *    accumulation; deterministic.  The weight gradient does not read the
 *    weights and is the same as with SNACK_BF16.  It needs the gathered
 *    activation's feature count (I for the forward, O for the input gradient)
 *    to be a multiple of 8 and that activation 16-byte aligned
 *    (SNACK_ERR_SHAPE / SNACK_ERR_ALIGN otherwise), and it is meant for
 *    batches of 32 and more (the matrix-core tiles are 32 batch rows wide).
 *    Every product of a dense tile includes the zeros of W: a NaN or infinite
 *    activation turns every output of its 64-key tile into NaN, as a dense
 *    product with a masked weight would.  All outputs are overwritten.
 *  - Preconditions on a descriptor (established by snack_coo_build, checked
 *    there, NOT re-checked by device calls): entries sorted by (row, col),
 *    unique, in range; row_offsets and the column view consistent with them.
 *    Device calls check only O(1) things (null pointers, sizes, dtype,
 *    workspace size).
 *  - Kernel choice: each device call picks its kernels from the layer's size,
 *    the batch and the value order; results agree to rounding whichever runs,
 *    and every kernel is deterministic except the batch-1 input gradient's
 *    LDS-atomic scatter (values in row order, at least 2^21 entries, and
 *    in_features above 10240 or vals / cols not 16-byte aligned).  Layers of
 *    at least 2^20 entries at batches padded to
 *    a multiple of 16 take LDS-tiled kernels (operand rows staged in LDS per
 *    column block, see row_blocks / col_blocks).  For tests and measurement,
 *    snack_coo_set_option overrides these choices process-wide (below).
 */
#ifndef SNACK_COO_H
#define SNACK_COO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum snack_status {
    SNACK_OK = 0,
    SNACK_ERR_NULL = 1,        /* a required pointer is NULL */
    SNACK_ERR_SHAPE = 2,       /* negative or inconsistent sizes, nnz > O*I, sizes beyond int32 */
    SNACK_ERR_INDEX = 3,       /* builder/topology: a row or column index out of range */
    SNACK_ERR_DUPLICATE = 4,   /* builder: a (row, col) pair appears twice */
    SNACK_ERR_ALIGN = 5,       /* a device pointer is not aligned to its element size */
    SNACK_ERR_DTYPE = 6,       /* unknown activation dtype or op code */
    SNACK_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than snack_coo_workspace_bytes */
    SNACK_ERR_HIP = 8,         /* a HIP launch failed (message has hipGetErrorString) */
    SNACK_ERR_INTERNAL = 9,    /* unexpected internal failure */
    SNACK_ERR_NOMEM = 10,      /* host allocation failed (builder / topology) */
    SNACK_ERR_UNSORTED = 11    /* topology: input triple not strictly sorted by (row, col) */
} snack_status;

enum { SNACK_F32 = 0, SNACK_BF16 = 1, SNACK_BF16_HW = 2 };               /* activation dtype */
enum { SNACK_OP_FWD = 0, SNACK_OP_BWD_INPUT = 1, SNACK_OP_GRAD_WEIGHT = 2, SNACK_OP_BWD = 3 };

/* A layer's weight on the device.  Every pointer is a DEVICE pointer,
 * borrowed for the duration of the call.
 *   rows, cols, vals   [nnz]  the triple, sorted by (row, col)
 *   row_offsets        [O+1]  row_offsets[r] = number of entries with row < r
 *                             (Table 7's CSR index pointer); required
 *   col_perm           [nnz]  column view: positions k of the triple listed in
 *                             (col, row) order (Table 7's CSC order)
 *   col_rows, col_cols [nnz]  rows[col_perm[j]], cols[col_perm[j]]
 *   col_offsets        [I+1]  col_offsets[c] = number of entries with col < c
 *   row_to_col         [nnz]  NULL, or the inverse of col_perm (row_to_col[col_perm[j]] = j;
 *                             see snack_coo_invert_perm).  Non-NULL selects VALUES IN
 *                             COLUMN ORDER: vals[j] is the value of column-view entry j
 *                             (of triple entry col_perm[j]), and every dW output is in the
 *                             same order (dW[j] for that entry).  The products are the same;
 *                             only the storage order of vals and dW changes.  It lets the
 *                             backward pass (a walk over the column view) read vals and
 *                             write dW contiguously, and moves one permuted read per entry
 *                             to the forward pass instead.  Requires the column view.
 *   row_blocks  [nb_r*O*4] NULL, or the row order cut into column blocks: nb_r =
 *                             ceil(I / 638) blocks of w_r = ceil(I / nb_r) columns.  For
 *                             block j and list position p, the four int32s at (j*O + p)*4 are
 *                             {r, start, end, 0}: row r's entries with a column in
 *                             [j*w_r, (j+1)*w_r) are the triple positions [start, end).  Each
 *                             (row, block) segment is the run of the row's entries whose
 *                             operand rows the tiled kernels stage together in LDS (Section
 *                             3.1's row-sorted triple makes it contiguous).  Within each
 *                             window of 32 positions [32w, 32w + 32) the rows are rows
 *                             32w .. 32w + 31, by decreasing end - start, equal lengths by
 *                             increasing row.  16-byte aligned.
 *   col_blocks  [nb_c*I*4] NULL, or the same for the column view: nb_c = ceil(O / 638)
 *                             blocks of w_c = ceil(O / nb_c) rows, positions in column-view
 *                             order.  Requires the column view.
 *                             Both tables depend on the structure only (not on the values or
 *                             their order); fill them with snack_coo_block_offsets.  When NULL,
 *                             a call that needs one builds it in its workspace (one extra
 *                             kernel per call).
 * The column view is needed by snack_coo_bwd_input and snack_coo_bwd, and with
 * row_to_col (NULL elsewhere). */
typedef struct snack_coo_desc {
    int64_t out_features;
    int64_t in_features;
    int64_t nnz;
    const int32_t *rows;
    const int32_t *cols;
    const float *vals;
    const int32_t *row_offsets;
    const int32_t *col_perm;
    const int32_t *col_rows;
    const int32_t *col_cols;
    const int32_t *col_offsets;
    const int32_t *row_to_col;
    const int32_t *row_blocks;
    const int32_t *col_blocks;
} snack_coo_desc;

/* Host-side COO builder (Appendix B, Table 7: COO triple, CSR index pointer,
 * CSC view; Section 3.1: the COO and CSR forms are interchangeable).
 * Inputs rows/cols/vals [nnz] are HOST arrays in any order.  Validates every
 * index (SNACK_ERR_INDEX), rejects repeated (row, col) pairs
 * (SNACK_ERR_DUPLICATE) and nnz > O*I or sizes beyond int32 (SNACK_ERR_SHAPE).
 * Outputs (HOST, caller-allocated; each may be NULL except rows_out and
 * cols_out when nnz > 0):
 *   rows_out, cols_out, vals_out [nnz]  the triple sorted by (row, col);
 *                                       vals are moved bit-exactly
 *   perm_out        [nnz]  input position of each sorted entry
 *   row_offsets_out [O+1]
 *   col_perm_out, col_rows_out, col_cols_out [nnz], col_offsets_out [I+1]:
 *                          the column view described at snack_coo_desc.
 * vals may be NULL only if vals_out is NULL.  Pure host code: no GPU needed. */
int snack_coo_build(int64_t out_features, int64_t in_features, int64_t nnz,
                    const int32_t *rows, const int32_t *cols, const float *vals,
                    int32_t *rows_out, int32_t *cols_out, float *vals_out,
                    int32_t *perm_out, int32_t *row_offsets_out,
                    int32_t *col_perm_out, int32_t *col_rows_out, int32_t *col_cols_out,
                    int32_t *col_offsets_out);

/* Bytes of device workspace that `op` (SNACK_OP_*) needs for this layer,
 * batch size and activation dtype.  0 is a valid answer.  Returns 0 with
 * snack_last_error() set if the arguments are invalid.  The answer can depend
 * on the descriptor's pointers (at batch 1 the input gradient of a large layer
 * takes its fastest kernel only when cols and vals are 16-byte aligned), so
 * ask again for a descriptor whose arrays moved. */
size_t snack_coo_workspace_bytes(int op, const snack_coo_desc *W, int64_t batch, int act_dtype);

/* Forward SNACK layer (Algorithm 1 with the nn.Linear bias of Section 3.5):
 * Y[b,o] = bias[o] + sum_{k: rows[k]=o} vals[k] X[b,cols[k]].
 *   X     device [batch][I], fp32 or bf16 (act_dtype)
 *   bias  device [O] fp32 or NULL (= 0); rows without entries output bias
 *   Y     device [batch][O], same dtype as X, overwritten
 *   workspace: device, >= snack_coo_workspace_bytes(SNACK_OP_FWD, ...) bytes,
 *   256-byte aligned.  batch may be 0 (no-op). */
int snack_coo_fwd(const snack_coo_desc *W, const void *X, int64_t batch, int act_dtype,
                  const float *bias, void *Y,
                  void *workspace, size_t workspace_bytes, void *hip_stream);

/* snack_coo_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and results, with the
 * workspace taken from a static device array of SNACK_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every device it runs on until the process ends.  The call allocates nothing; on its
 * first call on a device (with that device current) it looks up that device's copy of the array.
 * A call that needs more than SNACK_NOALLOC_SCRATCH_BYTES of workspace (snack_coo_workspace_bytes
 * with SNACK_OP_FWD) returns SNACK_ERR_WORKSPACE and launches nothing.  Every call on one device
 * shares the array: calls whose work overlaps on a device (other streams, other threads) race and
 * must be ordered by the caller. */
#define SNACK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int snack_coo_fwd_noalloc(const snack_coo_desc *W, const void *X, int64_t batch, int act_dtype,
                          const float *bias, void *Y, void *hip_stream);

/* Input gradient (Section 3.4 / Appendix F: dL/dX = W^T dL/dA, with W^T
 * obtained by swapping the row and column index arrays):
 * dX[b,i] = sum_{k: cols[k]=i} vals[k] dY[b,rows[k]].
 *   dY  device [batch][O], fp32 or bf16; dX device [batch][I], same dtype
 *   db  device [O] fp32 or NULL: if given, db[o] = sum_b dY[b,o] (the bias
 *       gradient of the nn.Linear drop-in)
 *   Requires the column view in W. */
int snack_coo_bwd_input(const snack_coo_desc *W, const void *dY, int64_t batch, int act_dtype,
                        void *dX, float *db,
                        void *workspace, size_t workspace_bytes, void *hip_stream);

/* Weight gradient on the support (Section 3.4 / Appendix F: sum of the batch's
 * rank-1 outer products evaluated only at (i,j) in supp(W)):
 * dW[k] = sum_b dY[b,rows[k]] X[b,cols[k]], written in the order of the
 * triple (in column-view order with row_to_col; fp32, overwritten; entries
 * with vals[k] == 0 are still computed).
 *   X device [batch][I], dY device [batch][O], fp32 or bf16; dW device [nnz]. */
int snack_coo_grad_weight(const snack_coo_desc *W, const void *X, const void *dY,
                          int64_t batch, int act_dtype, float *dW,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/* Both gradients of the backward pass (Section 3.4 / Appendix F: dL/dX and the
 * weight gradient on supp(W) are computed from the same upstream gradient):
 * the results of snack_coo_bwd_input (dX, and db if not NULL) and of
 * snack_coo_grad_weight (dW) in one call.  For batches 2..256 one pass over
 * the column view gathers each entry's dY row once for both products (the
 * feature-major copies are padded with zero columns to a batch tile of
 * 4*BT*Q columns, BT a power of two <= 16 and Q <= 4); at batch 1 and above
 * 256 the two operations run one after the other on the stream.  Arguments and layouts as for the
 * two calls; requires the column view; workspace >=
 * snack_coo_workspace_bytes(SNACK_OP_BWD, ...).  dX and dW are overwritten
 * (dW in the order of the triple, or of the column view with row_to_col);
 * results agree with the separate calls to rounding (the summation order of
 * dX differs).  Forms (snack_coo_bwd_is_fused tells which one a call takes):
 * with the tiled kernels applicable (see the conventions above) and one batch
 * tile (padded batch 16, 32 or 64), values in row order take two tiled passes
 * (the input gradient over the column view, then the weight gradient over the
 * row view, both reading X and dY in place), and values in column order one
 * tiled pass that serves each staged dY row to both gradients; otherwise the
 * one-pass kernel that gathers each entry's dY row from L2 once for both
 * gradients.  Layers of at least 2^20
 * entries take a row-banded form of that one-pass kernel: the rows are cut into
 * 8 bands of about nnz/8 entries, each band's part of every column is walked on
 * its own, and the 8 partial dX are added in band order (deterministic; the
 * workspace then also holds 8*I*Bp floats, Bp the padded batch; values in
 * column order never take the banded form).  SNACK_OPT_BAND_MIN_NNZ
 * (snack_coo_set_option) overrides that threshold. */
int snack_coo_bwd(const snack_coo_desc *W, const void *X, const void *dY, int64_t batch, int act_dtype,
                  void *dX, float *db, float *dW,
                  void *workspace, size_t workspace_bytes, void *hip_stream);

/* Whether snack_coo_bwd takes both gradients in one pass over the column view (1: the kernel that
 * gathers dY rows from L2, or the tiled pass that serves them from LDS), or in two passes (0: the
 * tiled input gradient over the column view and the tiled weight gradient over the row view, or at
 * batch 1 the two gradients' own kernels) for this weight, batch and dtype -- the choice the call
 * would make.  Negative: -(status) for an invalid descriptor.  For timing and diagnostics. */
int snack_coo_bwd_is_fused(const snack_coo_desc *W, int64_t batch, int act_dtype);

/* Device-side topology update (Appendix G prune-and-regrow, regrowth by
 * Algorithm 2): the same result as snack_coo_topology_update on the same
 * triple, n_prune and seed followed by snack_coo_build's column view, bit for
 * bit, computed on the GPU.  Input W: a device triple sorted strictly by
 * (row, col) with its values in row order (row_to_col NULL, else
 * SNACK_ERR_UNSORTED; as the builder emits; not re-checked), row offsets and
 * column view not needed.  Outputs (device, caller-owned, must not
 * alias W's arrays): rows_out, cols_out, vals_out [nnz], row_offsets_out
 * [O+1], col_perm_out, col_rows_out, col_cols_out [nnz], col_offsets_out
 * [I+1]; trials_out (HOST int64, or NULL) receives Algorithm 2's number of
 * draws.  The regrowth generates its draws in batches and reads back one count
 * per batch, so this call synchronizes hip_stream (it cannot be captured in a
 * graph).  workspace >= snack_coo_topology_workspace_bytes(O, I, nnz, n_prune),
 * 256-byte aligned.  O*I is limited to 2^34 positions. */
int snack_coo_topology_update_device(const snack_coo_desc *W, int64_t n_prune, uint64_t seed,
                                     int32_t *rows_out, int32_t *cols_out, float *vals_out,
                                     int32_t *row_offsets_out, int32_t *col_perm_out, int32_t *col_rows_out,
                                     int32_t *col_cols_out, int32_t *col_offsets_out, int64_t *trials_out,
                                     void *workspace, size_t workspace_bytes, void *hip_stream);

/* Bytes of device workspace snack_coo_topology_update_device needs (0 with
 * snack_last_error() set for invalid sizes).  SNACK_OPT_TOPOLOGY_DRAW_BATCH
 * (snack_coo_set_option) fixes the number of draws per batch, which is
 * otherwise sized from the expected number of draws. */
size_t snack_coo_topology_workspace_bytes(int64_t out_features, int64_t in_features, int64_t nnz,
                                          int64_t n_prune);

/* Host-side uniform initializer (Algorithm 2; its expected cost of about
 * -ln(eta)/(1-eta) trials per entry at sparsity eta is in Appendix F): nnz
 * distinct positions of the O x I matrix drawn by rejection.  Each trial draws
 * row = getrand(O), then col = getrand(I), with getrand(n) = floor(u * n / 2^64)
 * of the next SplitMix64 output u of a generator started at `seed` (the same
 * generator as the regrowth of snack_coo_topology_update), and keeps the pair
 * unless it was drawn before.  Output (host, caller-owned): rows_out, cols_out
 * [nnz] sorted by (row, col), row_offsets_out [O+1] or NULL, the number of
 * trials in trials_out (or NULL).  O*I is limited to 2^34 positions.  Values
 * are the caller's (the pages fix only the positions). */
int snack_coo_init_uniform(int64_t out_features, int64_t in_features, int64_t nnz, uint64_t seed,
                           int32_t *rows_out, int32_t *cols_out, int32_t *row_offsets_out,
                           int64_t *trials_out);

/* Host-side topology update (Appendix G: magnitude prune-and-regrow; regrowth
 * with the uniform initializer of Algorithm 2).  Input: a HOST triple sorted
 * strictly by (row, col) (SNACK_ERR_UNSORTED otherwise).
 *  1. prune the n_prune entries of smallest |vals| (ties: lower position first);
 *  2. regrow n_prune positions: draw row = getrand(O), then col = getrand(I),
 *     reject the pair if it is live (survivors and positions already regrown),
 *     where getrand(n) = floor(u * n / 2^64) of the next SplitMix64 output u
 *     of a generator started at `seed`; regrown entries get the value +0.0f;
 *  3. write the result sorted by (row, col) (rows_out, cols_out, vals_out
 *     [nnz], row_offsets_out [O+1] or NULL) and the number of draws to
 *     trials_out (or NULL).
 * O*I is limited to 2^34 positions (a bitmap of live positions is used).
 * Outputs must not alias the inputs. */
int snack_coo_topology_update(int64_t out_features, int64_t in_features, int64_t nnz,
                              const int32_t *rows, const int32_t *cols, const float *vals,
                              int64_t n_prune, uint64_t seed,
                              int32_t *rows_out, int32_t *cols_out, float *vals_out,
                              int32_t *row_offsets_out, int64_t *trials_out);

/* Device helpers for values kept in column order (snack_coo_desc.row_to_col).
 * All pointers are DEVICE pointers; n < 2^31; the work is enqueued on hip_stream.
 *   snack_coo_invert_perm: inv[perm[j]] = j for j < n.  perm must be a
 *     permutation of 0..n-1 (not checked: a repeated or out-of-range index
 *     writes out of bounds).  With perm = col_perm this gives row_to_col.
 *   snack_coo_gather_f32: dst[j] = src[idx[j]] for j < n (0 <= idx[j] < length
 *     of src, not checked).  Row-order values to column order:
 *     idx = col_perm; back: idx = row_to_col.  dst must not alias src.
 * Errors: SNACK_ERR_SHAPE (bad n), SNACK_ERR_NULL, SNACK_ERR_ALIGN (4 bytes). */
int snack_coo_invert_perm(const int32_t *perm, int64_t n, int32_t *inv, void *hip_stream);
int snack_coo_gather_f32(const float *src, const int32_t *idx, int64_t n, float *dst, void *hip_stream);

/* Timing probe for benchmarks and profilers (not part of the method).  While
 * armed on the calling thread, each device call records `start_event` on its
 * stream immediately before launching its main kernel (the gather-reduce of
 * snack_coo_fwd / snack_coo_bwd_input, the sampled product of
 * snack_coo_grad_weight, the fused pass of snack_coo_bwd) and `stop_event`
 * immediately after it, so the pair
 * brackets exactly that kernel.  Both are caller-owned hipEvent_t handles
 * created with timing enabled; passing NULL for both disarms the probe.
 * Returns SNACK_ERR_NULL if exactly one of them is NULL. */
int snack_coo_set_probe(void *start_event, void *stop_event);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *snack_last_error(void);

/* ABI version of this header: 10.  3 added snack_coo_init_uniform, 4 the device topology update,
 * 5 values in column order (snack_coo_desc.row_to_col, snack_coo_invert_perm, snack_coo_gather_f32),
 * 6 the segment tables (snack_coo_desc.row_blocks / col_blocks, snack_coo_block_offsets_count,
 * snack_coo_block_offsets), 7 the kernel-selection options (snack_coo_set_option,
 * snack_coo_get_option) in place of environment variables, 8 snack_coo_fwd_noalloc, 9 segment
 * tables as per-block lists of {key, start, end} ordered by length within windows of 32 keys,
 * 10 the half-precision path (act_dtype SNACK_BF16_HW) and SNACK_OPT_BF16_DW_MFMA. */
int snack_coo_abi_version(void);

/* Kernel-selection overrides for tests and measurement (not part of the method).  Process-wide,
 * read by every later call (snack_coo_workspace_bytes included); -1 restores the library's own
 * choice.  They pick among kernels that compute the same products, so results agree to
 * rounding whatever is set.
 *   SNACK_OPT_TILE                 0: no LDS-tiled kernels
 *   SNACK_OPT_BWD_FORM             form of snack_coo_bwd where more than one applies: 0 the one-pass
 *                                  kernel reading dY rows from L2, 1 two tiled passes, 2 one tiled pass
 *   SNACK_OPT_BAND_MIN_NNZ         entry count from which the one-pass backward runs in row bands
 *                                  (default 2^20)
 *   SNACK_OPT_TOPOLOGY_DRAW_BATCH  draws per batch of snack_coo_topology_update_device (>= 1)
 *   SNACK_OPT_BF16_DW_MFMA         the weight gradient with bf16 activations at batches of 256 and
 *                                  more on the matrix cores (dense products over the batch sampled
 *                                  at the stored entries): 1 wherever it applies, 0 never (default:
 *                                  layers at least 1/12 dense)
 * snack_coo_set_option returns SNACK_ERR_DTYPE for an unknown option and SNACK_ERR_SHAPE for a
 * value out of range; snack_coo_get_option returns the current value (-1 for an unknown option). */
enum {
    SNACK_OPT_TILE = 0,
    SNACK_OPT_BWD_FORM = 1,
    SNACK_OPT_BAND_MIN_NNZ = 2,
    SNACK_OPT_TOPOLOGY_DRAW_BATCH = 3,
    SNACK_OPT_BF16_DW_MFMA = 4
};
int snack_coo_set_option(int option, int64_t value);
int64_t snack_coo_get_option(int option);

/* Segment tables of snack_coo_desc.row_blocks (view = SNACK_VIEW_ROWS) and
 * snack_coo_desc.col_blocks (view = SNACK_VIEW_COLS): the number of int32
 * entries, nb * keys * 4 with keys = O and nb = ceil(I / 638) for the rows
 * (keys = I and nb = ceil(O / 638) for the column view; nb = 1 for an empty
 * dimension), or -1 with snack_last_error() set for a NULL descriptor or an
 * unknown view. */
enum { SNACK_VIEW_ROWS = 0, SNACK_VIEW_COLS = 1 };
int64_t snack_coo_block_offsets_count(const snack_coo_desc *W, int view);

/* Fills `out` (DEVICE, snack_coo_block_offsets_count entries, caller-owned)
 * with the segment table of one view, reading row_offsets and cols (rows) or
 * col_offsets and col_rows (column view) of W; enqueued on hip_stream.  The
 * table stays valid while the structure does: rebuild it after a topology
 * update.  Errors: SNACK_ERR_NULL (W, out or a needed array NULL),
 * SNACK_ERR_ALIGN (out not 16-byte aligned), SNACK_ERR_DTYPE (unknown view), SNACK_ERR_HIP. */
int snack_coo_block_offsets(const snack_coo_desc *W, int view, int32_t *out, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SNACK_COO_H */
