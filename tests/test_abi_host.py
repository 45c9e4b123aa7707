"""Host-side checks of the C ABI (no GPU needed).

libmsq.so must load, export every function include/msq.h declares, and refuse
bad arguments with the documented status codes before touching the GPU.
msq_plan is host-only and is exercised fully here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_wise_mixed_amd as msq
from block_wise_mixed_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, SHAPE, BITS, PERM, SMALL, HIP, UNSUP = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msq.library_path()):
        pytest.fail("libmsq.so is not built (run __graft_entry__.build())")
    return msq.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "msq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(msq_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"msq_plan", "msq_quantize_pack", "msq_gemm", "msq_gemm_ex",
            "msq_gemm_workspace_bytes", "msq_gemm_workspace_bytes_ex", "msq_gemm_group",
            "msq_gemm_group_ex", "msq_gemm_group_workspace_bytes_ex",
            "msq_status_string", "msq_format_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert lib.msq_status_string(s)
    assert lib.msq_status_string(99) == b"unknown status"
    assert lib.msq_format_version() == 2 == msq.FORMAT_VERSION


def _plan_raw(lib, N, K, bits, pr, pc):
    out = msq._Sizes()
    b = np.ascontiguousarray(bits, np.uint8)
    p = np.ascontiguousarray(pr, np.int32)
    q = np.ascontiguousarray(pc, np.int32)
    st = lib.msq_plan(N, K, b.ctypes.data, p.ctypes.data, q.ctypes.data, ctypes.byref(out))
    return st, out


def test_plan_sizes(lib):
    c = synth.random_case(256, 512, 0)
    st, out = _plan_raw(lib, 256, 512, c.bits, c.perm_row, c.perm_col)
    assert st == OK
    total = int(c.bits.astype(np.int64).sum())
    assert out.code_bytes == 1024 * total
    assert out.scale_bytes == 4 * 256 * 4 and out.zero_bytes == 256 * 4 and out.offset_bytes == 4 * 16
    hist = np.bincount(c.bits.ravel(), minlength=17)
    assert list(out.blocks_per_bits) == list(hist)
    assert out.mean_bits == pytest.approx(total / 16)


def test_plan_error_matrix(lib):
    c = synth.random_case(128, 256, 1)
    b, p, q = c.bits, c.perm_row, c.perm_col
    assert _plan_raw(lib, 100, 256, np.zeros(8, np.uint8), np.arange(100), q)[0] == SHAPE
    assert _plan_raw(lib, 128, 200, b, p, np.arange(200))[0] == SHAPE
    assert _plan_raw(lib, 0, 256, b, p, q)[0] == SHAPE
    assert _plan_raw(lib, -64, 256, b, p, q)[0] == SHAPE
    for bad in (5, 6, 7, 9, 255):
        bb = b.copy()
        bb[1, 1] = bad
        assert _plan_raw(lib, 128, 256, bb, p, q)[0] == BITS
    pp = p.copy()
    pp[3] = pp[4]
    assert _plan_raw(lib, 128, 256, b, pp, q)[0] == PERM
    qq = q.copy()
    qq[0] = 256
    assert _plan_raw(lib, 128, 256, b, p, qq)[0] == PERM
    qq[0] = -1
    assert _plan_raw(lib, 128, 256, b, p, qq)[0] == PERM
    out = msq._Sizes()
    out.code_bytes = 12345
    assert lib.msq_plan(128, 256, None, p.ctypes.data, q.ctypes.data, ctypes.byref(out)) == INVALID
    assert out.code_bytes == 12345  # untouched on error
    st, _ = _plan_raw(lib, 128, 256, b, p, q)
    assert st == OK


def test_plan_python_wrapper(lib):
    c = synth.random_case(64, 128, 2)
    sz = msq.plan(64, 128, c.bits, c.perm_row, c.perm_col)
    assert sz["code_bytes"] == 1024 * int(c.bits.sum())
    with pytest.raises(msq.MsqError):
        msq.plan(64, 128, np.full((1, 1), 7, np.uint8), c.perm_row, c.perm_col)


def _fake_weight(N=128, K=256, code_bytes=1 << 20):
    """Descriptor with aligned, non-null fake addresses: only argument checks may read it."""
    w = msq._Weight()
    w.N, w.K = N, K
    base = 1 << 40
    w.bits, w.perm_row, w.perm_col = base, base + 4096, base + 8192
    w.block_offset, w.codes, w.scale, w.zero = base + 12288, base + 16384, base + (1 << 30), base + (1 << 31)
    w.code_bytes = code_bytes
    return w


def _opt(kernel=0, **kw):
    o = msq._Options()
    o.kernel = kernel
    for k, v in kw.items():
        setattr(o, k, v)
    return ctypes.byref(o)


def test_gemm_argument_errors_before_any_launch(lib):
    w = _fake_weight()
    x, y, ws = 1 << 41, 1 << 42, 1 << 43
    g = lib.msq_gemm_ex
    big = 1 << 30
    assert g(x, 1, ctypes.byref(w), y, ws, big, _opt(7), None) == INVALID          # bad kernel enum
    assert g(x, 1, ctypes.byref(w), y, ws, big, _opt(gemv_waves=5), None) == INVALID
    assert g(x, 1, ctypes.byref(w), y, ws, big, _opt(gemv_split=-1), None) == INVALID
    assert g(x, 1, ctypes.byref(w), y, ws, big, _opt(gemm_split=-3), None) == INVALID
    assert g(x, 1, None, y, ws, big, None, None) == INVALID                         # null weight
    assert g(x, -1, ctypes.byref(w), y, ws, big, None, None) == SHAPE               # M < 0
    assert g(None, 0, ctypes.byref(w), None, None, 0, None, None) == OK             # M == 0: no-op
    assert g(None, 4, ctypes.byref(w), y, ws, big, None, None) == INVALID           # null x
    assert g(x + 2, 4, ctypes.byref(w), y, ws, big, None, None) == INVALID          # misaligned x
    assert g(x, 65, ctypes.byref(w), y, ws, big, _opt(1), None) == UNSUP            # GEMV with M > 64
    assert g(x, 600, ctypes.byref(w), y, ws, 1, _opt(2), None) == SMALL             # workspace too small
    assert g(x, 600, ctypes.byref(w), y, ws + 16, big, _opt(2), None) == INVALID    # misaligned workspace
    w2 = _fake_weight(N=100)
    assert g(x, 1, ctypes.byref(w2), y, ws, big, None, None) == SHAPE
    w3 = _fake_weight()
    w3.codes = (1 << 40) + 16400  # not 256-aligned
    assert g(x, 1, ctypes.byref(w3), y, ws, big, None, None) == INVALID
    w4 = _fake_weight()
    w4.scale = None
    assert lib.msq_gemm(x, 1, ctypes.byref(w4), y, ws, big, None) == INVALID


def test_options_workspace_sizes(lib):
    """msq_gemm_workspace_bytes_ex: NULL options = msq_gemm_workspace_bytes; forced K
    splits add their fp32 partials; bad options size nothing."""
    f = lib.msq_gemm_workspace_bytes_ex
    for M in (1, 16, 64, 2048):
        assert f(M, 4096, 14336, None) == lib.msq_gemm_workspace_bytes(M, 4096, 14336)
    auto1 = f(1, 4096, 8192, _opt(1))
    split8 = f(1, 4096, 8192, _opt(1, gemv_split=8))
    assert split8 >= 8 * 4096 * 4 and split8 > auto1
    g1 = f(130, 4096, 8192, _opt(2, gemm_split=1))
    g4 = f(130, 4096, 8192, _opt(2, gemm_split=4))
    assert g4 - g1 >= 4 * 130 * 4096 * 4
    assert f(1, 4096, 8192, _opt(gemv_waves=3)) == 0
    assert f(1, 4096, 8192, _opt(9)) == 0


def test_quantize_pack_argument_errors_before_any_launch(lib):
    w = _fake_weight()
    assert lib.msq_quantize_pack(None, ctypes.byref(w), None) == INVALID
    assert lib.msq_quantize_pack((1 << 41) + 2, ctypes.byref(w), None) == INVALID
    assert lib.msq_quantize_pack(1 << 41, None, None) == INVALID
    w2 = _fake_weight(K=100)
    assert lib.msq_quantize_pack(1 << 41, ctypes.byref(w2), None) == SHAPE


def test_workspace_sizes(lib):
    assert lib.msq_gemm_workspace_bytes(0, 4096, 4096) == 0
    assert lib.msq_gemm_workspace_bytes(1, 100, 4096) == 0
    for M in (1, 16, 64, 65, 2048):
        ws = lib.msq_gemm_workspace_bytes(M, 4096, 14336)
        # at least the gathered activations and group sums the prefill kernel stages
        assert ws >= M * 14336 * 2 + M * 112 * 4


def _group_arrays(ws_list):
    arr = (ctypes.POINTER(msq._Weight) * len(ws_list))(*[ctypes.pointer(w) for w in ws_list])
    return arr


def test_group_argument_errors_before_any_launch(lib):
    ws_list = [_fake_weight(), _fake_weight(N=256, K=512)]
    arr = _group_arrays(ws_list)
    xs = (ctypes.c_void_p * 2)(1 << 41, 1 << 41)
    ys = (ctypes.c_void_p * 2)(1 << 42, (1 << 42) + 4096)
    ws = 1 << 43
    g = lib.msq_gemm_group
    assert g(xs, 1, arr, ys, 0, ws, 1 << 30, None) == INVALID      # count 0
    assert g(xs, 1, arr, ys, 9, ws, 1 << 30, None) == INVALID      # count > MSQ_GROUP_MAX
    assert g(None, 1, arr, ys, 2, ws, 1 << 30, None) == INVALID    # null array
    assert g(xs, -1, arr, ys, 2, ws, 1 << 30, None) == SHAPE       # M < 0
    assert g(xs, 0, arr, ys, 2, None, 0, None) == OK              # M == 0: no-op
    assert g(xs, 1, arr, ys, 2, ws, 1, None) == SMALL              # workspace too small
    assert g(xs, 1, arr, ys, 2, ws + 16, 1 << 30, None) == INVALID  # misaligned workspace
    bad_x = (ctypes.c_void_p * 2)(1 << 41, (1 << 41) + 2)
    assert g(bad_x, 1, arr, ys, 2, ws, 1 << 30, None) == INVALID   # misaligned second x
    arr_bad = _group_arrays([_fake_weight(), _fake_weight(K=100)])
    assert g(xs, 1, arr_bad, ys, 2, ws, 1 << 30, None) == SHAPE    # bad second shape


def test_group_workspace_sizes(lib):
    ws_list = [_fake_weight(N=4096, K=4096), _fake_weight(N=1024, K=4096), _fake_weight(N=8192, K=14336)]
    arr = _group_arrays(ws_list)
    singles = [lib.msq_gemm_workspace_bytes(1, w.N, w.K) for w in ws_list]
    # M == 1: every matrix keeps its own activation prep (reordered x, group sums,
    # corrections) and partials; the group's K splits are no more than a single
    # call's (the split count is planned for the whole launch)
    prep = sum(2 * w.K + 84 * (w.K // 128) for w in ws_list)
    g1 = lib.msq_gemm_group_workspace_bytes(1, arr, 3)
    assert prep <= g1 <= sum(singles) + 3 * 256
    # M in 2 .. 32: one gather and one decode launch for all, each matrix
    # with its own gathered activation; the group's K splits are no more than a
    # single call's
    mid = [lib.msq_gemm_workspace_bytes_ex(16, w.N, w.K, _opt(0)) for w in ws_list]
    g16 = lib.msq_gemm_group_workspace_bytes(16, arr, 3)
    assert sum(16 * w.K * 2 for w in ws_list) <= g16 <= sum(mid) + 3 * 256
    # prefill: one launch for all, each matrix with its own gathered activation
    big = [lib.msq_gemm_workspace_bytes(2048, w.N, w.K) for w in ws_list]
    g = lib.msq_gemm_group_workspace_bytes(2048, arr, 3)
    assert sum(big) <= g <= sum(big) + 3 * 256
    assert g >= sum(2048 * w.K * 2 for w in ws_list)
    assert lib.msq_gemm_group_workspace_bytes(0, arr, 3) == 0
    assert lib.msq_gemm_group_workspace_bytes(1, arr, 0) == 0
    assert lib.msq_gemm_group_workspace_bytes(1, arr, 9) == 0


def _hip_devices() -> int:
    """GPUs the HIP runtime sees (0 here on a host without one)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return 0
    n = ctypes.c_int(0)
    return n.value if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 else 0


def test_alloc_host_checks(lib):
    """Bit allocation: workspace sizing and argument checks, before any GPU work."""
    import ctypes
    lib.msq_alloc_workspace_bytes.restype = ctypes.c_size_t
    lib.msq_alloc_workspace_bytes.argtypes = [ctypes.c_int64]
    assert lib.msq_alloc_workspace_bytes(0) == 0
    assert lib.msq_alloc_workspace_bytes((1 << 28) + 1) == 0
    # hipCUB sizes its scan storage for the current device: with no device the
    # query fails and the size is refused (0), and so is the call
    gpu = _hip_devices() > 0
    if gpu:
        assert lib.msq_alloc_workspace_bytes(1000) >= 6 * 4 * 1000 + 1000
    else:
        assert lib.msq_alloc_workspace_bytes(1000) == 0
    f = lib.msq_allocate_bits
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 10, 5, None, None, 0, None, None) == 1          # null pointers
    assert f(256, 10, 5, 256, 257, 1 << 20, None, None) == 1       # misaligned workspace
    assert f(256, 0, 5, 256, 256, 1 << 20, None, None) == 2        # no blocks
    assert f(256, 10, -1, 256, 256, 1 << 20, None, None) == 2      # negative budget
    assert f(256, 10, 5, 256, 256, 16, None, None) == (5 if gpu else 6)  # too small / no device


def test_reorder_host_checks(lib):
    """Channel reordering: workspace sizing and argument checks, before any GPU work."""
    import ctypes
    lib.msq_reorder_workspace_bytes.restype = ctypes.c_size_t
    lib.msq_reorder_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
    assert lib.msq_reorder_workspace_bytes(64, 100) == 0        # K not a multiple of 128
    assert lib.msq_reorder_workspace_bytes(0, 128) == 0
    assert lib.msq_reorder_workspace_bytes(64, 65536) == 0      # K above the LDS limit
    assert lib.msq_reorder_workspace_bytes(256, 512) >= 4 * (256 + 512)
    f = lib.msq_reorder_channels
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, 64, 128, 1, 256, 256, 256, 1 << 20, None) == 1
    assert f(264, 64, 128, 1, 256, 256, 256, 1 << 20, None) == 1   # saliency not 16-byte aligned
    assert f(256, 65, 128, 1, 256, 256, 256, 1 << 20, None) == 2
    assert f(256, 64, 128, 1, 256, 256, 256, 16, None) == 5


def test_plan_counts_passthrough_blocks(lib):
    """16-bit blocks are accepted, counted and sized at 16 KiB each; other values are not."""
    c = synth.random_case(128, 256, 4, dist={16: .5, 2: .5})
    st, out = _plan_raw(lib, 128, 256, c.bits, c.perm_row, c.perm_col)
    assert st == OK
    assert out.blocks_per_bits[16] == int((c.bits == 16).sum()) > 0
    assert out.code_bytes == 1024 * int(c.bits.astype(np.int64).sum())
    for bad in (5, 6, 7, 9, 15, 17, 32):
        st, _ = _plan_raw(lib, 128, 256, np.full_like(c.bits, bad), c.perm_row, c.perm_col)
        assert st == 3


def test_negative_passthrough_count_rejected(lib):
    w = _fake_weight()
    w.tile16_blocks = -1
    x = 1 << 41
    assert lib.msq_gemm(x, 1, ctypes.byref(w), x, x, 1 << 30, None) == INVALID
