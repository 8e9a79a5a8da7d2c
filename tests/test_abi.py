"""The C-ABI library loads and exports every function include/snack_coo.h declares (CPU only)."""
import ctypes
import os
import re

import coo_spmm_row_amd as snk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "snack_coo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(snack_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 21, names
    lib = ctypes.CDLL(snk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(snk.EXPORTED)


def test_abi_version():
    """The version the header documents is the one the library reports."""
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                            "snack_coo.h")).read()
    m = re.search(r"ABI version of this header: (\d+)", hdr)
    assert m, "header states no ABI version"
    assert snk.abi_version() == int(m.group(1)) == 10


def test_binding_loads_only_the_in_tree_library():
    assert os.path.dirname(snk.LIB_PATH) == os.path.join(ROOT, "coo_spmm_row_amd")
    assert os.path.exists(snk.LIB_PATH)


def test_device_calls_reject_bad_arguments_before_any_launch():
    """Host-forced failures: the status comes back without touching a GPU."""
    lib = snk._lib
    assert lib.snack_coo_fwd(None, None, 1, 0, None, None, None, 0, None) == 1  # NULL descriptor
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 4, 4, 20  # nnz > O*I
    assert lib.snack_coo_fwd(ctypes.byref(d), None, 1, 0, None, None, None, 0, None) == 2
    assert b"nnz" in lib.snack_last_error()
    d.nnz = 0
    d.row_offsets = 0x1000
    assert lib.snack_coo_fwd(ctypes.byref(d), None, 1, 7, None, None, None, 0, None) == 6  # dtype
    assert lib.snack_coo_fwd(ctypes.byref(d), None, -1, 0, None, None, None, 0, None) == 2  # batch
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1000, 1, 0, None, None, None, 0, None) == 1  # Y NULL
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1001, 1, 0, None, 0x2000, None, 0, None) == 5  # misaligned X
    # bwd_input needs the column view
    d.nnz = 3
    d.rows = d.cols = d.vals = 0x1000
    assert lib.snack_coo_bwd_input(ctypes.byref(d), 0x1000, 1, 0, 0x1000, None, None, 0, None) == 1
    # a too-small workspace
    d.nnz = 3
    need = lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 8, 0)
    assert need > 0
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1000, 8, 0, None, 0x2000, 0x10000, need - 1, None) == 7
    assert lib.snack_coo_workspace_bytes(9, ctypes.byref(d), 8, 0) == 0
    # the fused backward: NULL descriptor, no column view, bad dtype, too-small workspace
    assert lib.snack_coo_bwd(None, None, None, 16, 0, None, None, None, None, 0, None) == 1
    assert lib.snack_coo_bwd(ctypes.byref(d), 0x1000, 0x1000, 16, 0, 0x1000, None, 0x1000, None, 0, None) == 1
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    assert lib.snack_coo_bwd(ctypes.byref(d), 0x1000, 0x1000, 16, 5, 0x1000, None, 0x1000, None, 0, None) == 6
    need = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 16, 0)
    assert need > 0
    assert lib.snack_coo_bwd(ctypes.byref(d), 0x1000, 0x1000, 16, 0, 0x1000, None, 0x1000, 0x10000, need - 1,
                             None) == 7
    assert lib.snack_coo_bwd(ctypes.byref(d), 0x1000, 0x1000, 16, 0, 0x1000, None, None, 0x10000, need,
                             None) == 1  # dW NULL


def test_noalloc_forward_rejects_before_any_launch():
    """snack_coo_fwd_noalloc: invalid arguments come back as from snack_coo_fwd, and a call whose
    workspace would exceed the static scratch returns SNACK_ERR_WORKSPACE (no GPU touched)."""
    lib = snk._lib
    assert lib.snack_coo_fwd_noalloc(None, None, 1, 0, None, None, None) == 1  # NULL descriptor
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 4, 4, 20  # nnz > O*I
    assert lib.snack_coo_fwd_noalloc(ctypes.byref(d), None, 1, 0, None, None, None) == 2
    d.out_features, d.in_features, d.nnz = 300, 100_000, 3
    d.rows = d.cols = d.vals = d.row_offsets = 0x1000
    need = lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 256, 0)
    assert need > snk.NOALLOC_SCRATCH_BYTES
    assert lib.snack_coo_fwd_noalloc(ctypes.byref(d), 0x1000, 256, 0, None, 0x2000, None) == 7
    assert b"static scratch" in lib.snack_last_error()


def test_one_hip_runtime_in_process():
    """The library binds to torch's HIP runtime (same soname), so torch streams and events are valid."""
    runtimes = snk._hip_runtimes_mapped()
    assert len(runtimes) == 1, runtimes


def test_banded_backward_workspace_follows_threshold():
    """The row-banded backward needs 8*I*B more floats of workspace; SNACK_OPT_BAND_MIN_NNZ moves the
    entry count from which snack_coo_bwd (and its workspace size) takes that form."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 300, 200, 5000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000  # host-side sizing only: never dereferenced
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    with snk.option(snk.OPT_BAND_MIN_NNZ, 1):
        banded = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, 0)
    with snk.option(snk.OPT_BAND_MIN_NNZ, 1 << 62):
        plain = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, 0)
    default = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, 0)  # 5000 < 2^20: not banded
    assert plain == default > 0
    assert banded - plain >= 8 * 200 * 64 * 4


def test_options_validated_and_restored():
    """snack_coo_set_option rejects unknown options and out-of-range values (the old value stays),
    and -1 restores the library's own choice."""
    lib = snk._lib
    for opt in (snk.OPT_TILE, snk.OPT_BWD_FORM, snk.OPT_BAND_MIN_NNZ, snk.OPT_TOPOLOGY_DRAW_BATCH,
                snk.OPT_BF16_DW_MFMA):
        assert snk.get_option(opt) == -1
    assert lib.snack_coo_set_option(9, 0) == 6 and lib.snack_coo_set_option(-1, 0) == 6  # SNACK_ERR_DTYPE
    for opt, bad in ((snk.OPT_TILE, 1), (snk.OPT_BWD_FORM, 3), (snk.OPT_BAND_MIN_NNZ, -2),
                     (snk.OPT_TOPOLOGY_DRAW_BATCH, 0), (snk.OPT_BF16_DW_MFMA, 2)):
        assert lib.snack_coo_set_option(opt, bad) == 2 and snk.get_option(opt) == -1  # SNACK_ERR_SHAPE
    with snk.option(snk.OPT_BWD_FORM, 2):
        assert snk.get_option(snk.OPT_BWD_FORM) == 2
    assert snk.get_option(snk.OPT_BWD_FORM) == -1
    assert lib.snack_coo_get_option(17) == -1



def test_column_order_values_host_checks_and_workspace():
    """Values in column order (row_to_col set): every device call then needs the column view, the
    weight gradient reserves nnz more floats of workspace for its row-order staging, the fused
    backward drops the row bands, and the device topology update refuses the layout."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 300, 200, 5000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000  # host-side sizing only: never dereferenced
    row_dw = lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 64, 0)
    d.row_to_col = 0x1000
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1000, 8, 0, None, 0x2000, 0x10000, 1 << 30, None) == 1
    assert b"column view" in lib.snack_last_error()
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 64, 0) >= row_dw + 4 * 5000
    d.nnz = 1 << 21
    d.out_features = d.in_features = 4096
    with snk.option(snk.OPT_BWD_FORM, 0):  # the one-pass kernel that gathers dY from L2
        col_bwd = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, 0)
        d.row_to_col = None
        row_bwd = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, 0)  # 2^21 entries: banded
    assert row_bwd - col_bwd >= 8 * 4096 * 64 * 4
    d.row_to_col = 0x1000
    ws = lib.snack_coo_topology_workspace_bytes(4096, 4096, 1 << 21, 10)
    assert lib.snack_coo_topology_update_device(ctypes.byref(d), 10, 0, *([0x1000] * 8), None, 0x10000, ws,
                                                None) == 11
    assert lib.snack_coo_invert_perm(None, 4, None, None) == 1
    assert lib.snack_coo_invert_perm(0x1000, -1, 0x1000, None) == 2
    assert lib.snack_coo_gather_f32(0x1001, 0x1000, 4, 0x1000, None) == 5
    assert lib.snack_coo_gather_f32(None, None, 0, None, None) == 0


def test_block_offsets_count_and_errors():
    """Segment-list sizes: ceil(n / 638) blocks * keys * 4 int32s; argument errors come back before any
    launch."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 10000, 10000, 0
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), snk.SNACK_VIEW_ROWS) == 16 * 10000 * 4
    d.out_features, d.in_features = 700, 638
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), snk.SNACK_VIEW_ROWS) == 1 * 700 * 4
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), snk.SNACK_VIEW_COLS) == 2 * 638 * 4
    d.in_features = 639
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), snk.SNACK_VIEW_ROWS) == 2 * 700 * 4
    d.in_features = 0
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), snk.SNACK_VIEW_ROWS) == 1 * 700 * 4
    assert lib.snack_coo_block_offsets_count(ctypes.byref(d), 5) == -1
    assert lib.snack_coo_block_offsets_count(None, 0) == -1
    d.in_features = 640
    d.row_offsets = 0x1000
    assert lib.snack_coo_block_offsets(ctypes.byref(d), 5, 0x1000, None) == 6      # unknown view
    assert lib.snack_coo_block_offsets(ctypes.byref(d), 0, None, None) == 1        # out NULL
    assert lib.snack_coo_block_offsets(ctypes.byref(d), 0, 0x1008, None) == 5      # out misaligned
    assert lib.snack_coo_block_offsets(ctypes.byref(d), 1, 0x1000, None) == 1      # no column view
    assert lib.snack_coo_block_offsets(None, 0, 0x1000, None) == 1


def test_tiled_workspace_bounded_by_batch_tiles():
    """The tiled kernels (and their block partials, batch x column blocks x keys floats) apply up to
    4096 batch columns; wider batches keep the wide-batch paths, whose workspace does not grow with
    the number of column blocks (host-side sizing only)."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 5000, 5000, 2_500_000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000
    nb = -(-5000 // 638)  # column blocks of the tiled walk
    for B in (256, 4096):
        fwd = lib.snack_coo_workspace_bytes(0, ctypes.byref(d), B, 0)
        assert fwd >= 4 * B * nb * 5000  # block partials of the tiled forward
    fwd8192 = lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 8192, 0)
    assert fwd8192 < 4 * 8192 * nb * 5000  # no partials: not tiled
    assert fwd8192 <= 4 * 5001 * 8192 + 4 * 2_500_000 + (1 << 20)  # operand copy and gathered values


def test_tiled_planner_entry_bound():
    """The tiled walks take 32-bit byte offsets into the per-entry arrays: a layer of 2^29 - 1
    entries takes them (block partials in the forward's workspace), one of 2^29 does not (host-side
    sizing only)."""
    lib = snk._lib
    d = snk._Desc()
    n = 1 << 16
    d.out_features, d.in_features = n, n
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000
    nb = -(-n // 638)
    partials = 4 * 64 * nb * n
    d.nnz = (1 << 29) - 1
    assert lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 64, 0) >= partials
    d.nnz = 1 << 29
    assert 0 < lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 64, 0) < partials


def test_backward_form_rules():
    """The documented choice of snack_coo_bwd's form (host-side planning, no GPU): two tiled passes
    for values in row order at one batch tile of 16, 32 or 64 columns on layers of >= 2^20 entries,
    two untiled passes at batch 1, one pass otherwise (the tiled pass for column order at one batch
    tile, the L2-gather kernel else); SNACK_OPT_TILE and SNACK_OPT_BWD_FORM override."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 10000, 10000, 5_000_000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    fused = lambda B: lib.snack_coo_bwd_is_fused(ctypes.byref(d), B, 0)
    # batch 1: the two gradients' own kernels one after the other (two passes, not tiled)
    assert [fused(B) for B in (1, 16, 32, 50, 64, 96, 128)] == [0, 0, 0, 0, 0, 1, 1]
    d.row_to_col = 0x1000  # values in column order: always one pass
    assert [fused(B) for B in (16, 64, 128)] == [1, 1, 1]
    d.row_to_col = None
    d.nnz = 1_000_000  # below 2^20 entries: never tiled
    assert fused(64) == 1
    d.nnz = 5_000_000
    for (opt, val), want in (((snk.OPT_TILE, 0), 1), ((snk.OPT_BWD_FORM, 0), 1), ((snk.OPT_BWD_FORM, 2), 1),
                             ((snk.OPT_BWD_FORM, 1), 0)):
        with snk.option(opt, val):
            assert fused(64) == want, (opt, val)


def test_backward_shared_copies_workspace():
    """On an untiled layer at a wide batch where both gradients take the row-wave kernels (a
    GPT-2-shaped 768 -> 3072 layer at batch 1024), snack_coo_bwd makes the feature-major copies of
    X and dY once, in the weight gradient's workspace, beside the input gradient's own: its
    workspace is at least the two separate calls' together, and holds both copies."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 3072, 768, 23593
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000  # host-side sizing only: never dereferenced
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    for B in (512, 1024):
        assert lib.snack_coo_bwd_is_fused(ctypes.byref(d), B, 0) == 0
        bwd = lib.snack_coo_workspace_bytes(3, ctypes.byref(d), B, 0)
        dx = lib.snack_coo_workspace_bytes(1, ctypes.byref(d), B, 0)
        dw = lib.snack_coo_workspace_bytes(2, ctypes.byref(d), B, 0)
        assert dw >= 4 * B * ((768 + 1) + (3072 + 1))  # X and dY feature-major, zero rows included
        assert bwd >= dx + dw


def test_half_precision_host_checks_and_workspace():
    """SNACK_BF16_HW (2): accepted by every device call and the workspace query, checked before any
    launch (gathered feature count a multiple of 8, activations 16-byte aligned), never the fused
    backward; its workspace holds the K groups' partial tiles (10k x 10k at batch 64: 4 groups of
    10000 x 64 fp32) and, without the descriptor's tables, the segment lists."""
    lib = snk._lib
    HW = snk.SNACK_BF16_HW
    assert HW == 2
    d = snk._Desc()
    d.out_features, d.in_features, d.nnz = 10000, 10000, 5_000_000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000  # host-side sizing and checks only
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    tables = 10000 * 16 * 16  # keys x blocks x 16 bytes
    part = 4 * 10000 * 64 * 4
    assert lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 64, HW) == part + tables
    d.row_blocks = d.col_blocks = 0x1000
    assert lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 64, HW) == part
    assert lib.snack_coo_workspace_bytes(1, ctypes.byref(d), 64, HW) == part
    assert lib.snack_coo_workspace_bytes(3, ctypes.byref(d), 64, HW) >= part
    assert lib.snack_coo_workspace_bytes(0, ctypes.byref(d), 64, 3) == 0  # unknown dtype
    assert lib.snack_coo_bwd_is_fused(ctypes.byref(d), 64, HW) == 0
    # I = 10000 is a multiple of 8; X 8- but not 16-byte aligned
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1008, 64, HW, None, 0x2000, 0x10000, 1 << 30, None) == 5
    assert b"16-byte" in lib.snack_last_error()
    d.in_features = 9996  # not a multiple of 8
    assert lib.snack_coo_fwd(ctypes.byref(d), 0x1000, 64, HW, None, 0x2000, 0x10000, 1 << 30, None) == 2
    assert b"multiple of 8" in lib.snack_last_error()
    d.in_features, d.out_features = 10000, 9996  # the input gradient gathers over O
    assert lib.snack_coo_bwd_input(ctypes.byref(d), 0x1000, 64, HW, 0x2000, None, 0x10000, 1 << 30, None) == 2
    assert lib.snack_coo_bwd(ctypes.byref(d), 0x1000, 0x1000, 64, HW, 0x2000, None, 0x3000, 0x10000, 1 << 30,
                             None) == 2


def test_bf16_weight_gradient_mfma_workspace_follows_rule():
    """The bf16 weight gradient on the matrix cores is planned for batches of 256 and more on
    layers at least 1/12 dense (or wherever SNACK_OPT_BF16_DW_MFMA = 1), its workspace then the two
    feature-major bf16 copies (plus the segment lists when the descriptor has none)."""
    lib = snk._lib
    d = snk._Desc()
    d.out_features, d.in_features = 5000, 5000
    d.row_offsets = d.rows = d.cols = d.vals = 0x1000  # host-side sizing only
    d.col_perm = d.col_rows = d.col_cols = d.col_offsets = 0x1000
    d.row_blocks = d.col_blocks = 0x1000
    copies = (5000 * 4096 * 2) * 2
    for code in (snk.SNACK_BF16, snk.SNACK_BF16_HW):
        d.nnz = 2_500_000  # 10 %: on the matrix cores
        assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 4096, code) == copies
        d.nnz = 1_250_000  # 5 %: the VALU kernels
        assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 4096, code) != copies
        with snk.option(snk.OPT_BF16_DW_MFMA, 1):
            assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 4096, code) == copies
            assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 255, code) != (5000 * 256 * 2) * 2
        d.nnz = 2_500_000
        with snk.option(snk.OPT_BF16_DW_MFMA, 0):
            assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 4096, code) != copies
    d.nnz = 2_500_000
    assert lib.snack_coo_workspace_bytes(2, ctypes.byref(d), 4096, snk.SNACK_F32) != copies  # fp32: never
