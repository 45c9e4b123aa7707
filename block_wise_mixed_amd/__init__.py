"""Block-wise mixed-precision weight-only quantized matmul for MI355X (gfx950).

Thin ctypes binding over the C ABI of libmsq.so (include/msq.h).  This module
only marshals arguments: every step of quantize-pack and of y = x . W^T runs
in the library's HIP kernels.  PyTorch provides device memory and the current
stream.  There is no fallback: if libmsq.so is missing every call raises.

    pw = quantize_pack(W_bf16_cuda, bits, perm_row, perm_col)   # offline
    y  = gemm(x_bf16_cuda, pw)                                   # fp32 [M][N]

Method: a bf16 weight is reordered in rows and columns, cut into 64x128
blocks with a bitwidth from {0,1,2,3,4,8} each, and every block row-group of
128 is round-to-nearest quantized with its own scale and zero point
("ScaleBITS" summary page, sections Approach and Limitations).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["MsqError", "PackedWeight", "plan", "quantize_pack", "allocate_packed", "pack_into",
           "pack_bytes", "gemm", "workspace_bytes",
           "OPTION_FIELDS", "gemm_noalloc", "NOALLOC_SCRATCH_BYTES",
           "gemm_group", "group_workspace_bytes", "GROUP_MAX",
           "library_path", "load_library", "KERNELS", "FORMAT_VERSION", "GEMV_MAX_M",
           "allocate_bits", "alloc_workspace_bytes", "ALLOC_LEVELS", "reorder_channels"]

FORMAT_VERSION = 2
GEMV_MAX_M = 64
KERNELS = {"auto": 0, "gemv": 1, "gemm": 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmsq.so"
_lib = None


def library_path() -> str:
    return os.environ.get("MSQ_LIBRARY", os.path.join(_HERE, _LIB_NAME))


class MsqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = _lib.msq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: msq status {status} ({text})")


class _Sizes(ctypes.Structure):
    _fields_ = [("code_bytes", ctypes.c_int64), ("scale_bytes", ctypes.c_int64),
                ("zero_bytes", ctypes.c_int64), ("offset_bytes", ctypes.c_int64),
                ("blocks_per_bits", ctypes.c_int64 * 17), ("mean_bits", ctypes.c_double)]


class _Options(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("gemv_split", ctypes.c_int32),
                ("gemv_waves", ctypes.c_int32), ("m1_prep", ctypes.c_int32),
                ("gemm_split", ctypes.c_int32)]


OPTION_FIELDS = ("gemv_split", "gemv_waves", "m1_prep", "gemm_split")


def _options(kernel: str = "auto", options: Optional[dict] = None) -> Optional[_Options]:
    """msq_options for a kernel name and a dict of launch choices (None: automatic)."""
    if kernel == "auto" and not options:
        return None
    o = _Options()
    o.kernel = KERNELS[kernel]
    for k, v in (options or {}).items():
        if k not in OPTION_FIELDS:
            raise ValueError(f"unknown option {k!r}; known: {OPTION_FIELDS}")
        setattr(o, k, int(v))
    return o


class _Weight(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("bits", ctypes.c_void_p), ("perm_row", ctypes.c_void_p),
                ("perm_col", ctypes.c_void_p), ("block_offset", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("zero", ctypes.c_void_p), ("code_bytes", ctypes.c_int64),
                ("tile16_blocks", ctypes.c_int64)]


def load_library():
    """Load libmsq.so once; raises OSError with the path if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise OSError(f"{path} not found: build it with `python -m block_wise_mixed_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.msq_plan.argtypes = [i64, i64, vp, vp, vp, ctypes.POINTER(_Sizes)]
    lib.msq_plan.restype = ctypes.c_int
    lib.msq_quantize_pack.argtypes = [vp, ctypes.POINTER(_Weight), vp]
    lib.msq_quantize_pack.restype = ctypes.c_int
    lib.msq_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    lib.msq_gemm_workspace_bytes.restype = sz
    lib.msq_gemm.argtypes = [vp, i64, ctypes.POINTER(_Weight), vp, vp, sz, vp]
    lib.msq_gemm.restype = ctypes.c_int
    lib.msq_gemm_ex.argtypes = [vp, i64, ctypes.POINTER(_Weight), vp, vp, sz,
                                ctypes.POINTER(_Options), vp]
    lib.msq_gemm_ex.restype = ctypes.c_int
    lib.msq_gemm_workspace_bytes_ex.argtypes = [i64, i64, i64, ctypes.POINTER(_Options)]
    lib.msq_gemm_workspace_bytes_ex.restype = sz
    lib.msq_gemm_group_workspace_bytes.argtypes = [i64, ctypes.POINTER(ctypes.POINTER(_Weight)),
                                                   ctypes.c_int]
    lib.msq_gemm_group_workspace_bytes.restype = sz
    lib.msq_gemm_group.argtypes = [ctypes.POINTER(vp), i64, ctypes.POINTER(ctypes.POINTER(_Weight)),
                                   ctypes.POINTER(vp), ctypes.c_int, vp, sz, vp]
    lib.msq_gemm_group.restype = ctypes.c_int
    lib.msq_gemm_group_workspace_bytes_ex.argtypes = [
        i64, ctypes.POINTER(ctypes.POINTER(_Weight)), ctypes.c_int, ctypes.POINTER(_Options)]
    lib.msq_gemm_group_workspace_bytes_ex.restype = sz
    lib.msq_gemm_group_ex.argtypes = [ctypes.POINTER(vp), i64,
                                      ctypes.POINTER(ctypes.POINTER(_Weight)), ctypes.POINTER(vp),
                                      ctypes.c_int, vp, sz, ctypes.POINTER(_Options), vp]
    lib.msq_gemm_group_ex.restype = ctypes.c_int
    lib.msq_alloc_workspace_bytes.argtypes = [i64]
    lib.msq_alloc_workspace_bytes.restype = sz
    lib.msq_allocate_bits.argtypes = [vp, i64, i64, vp, vp, sz, ctypes.POINTER(ctypes.c_int32), vp]
    lib.msq_allocate_bits.restype = ctypes.c_int
    lib.msq_reorder_workspace_bytes.argtypes = [i64, i64]
    lib.msq_reorder_workspace_bytes.restype = sz
    lib.msq_reorder_channels.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.msq_reorder_channels.restype = ctypes.c_int
    lib.msq_gemm_noalloc.argtypes = [vp, i64, ctypes.POINTER(_Weight), vp, vp]
    lib.msq_gemm_noalloc.restype = ctypes.c_int
    lib.msq_status_string.argtypes = [ctypes.c_int]
    lib.msq_status_string.restype = ctypes.c_char_p
    lib.msq_format_version.argtypes = []
    lib.msq_format_version.restype = ctypes.c_int
    if lib.msq_format_version() != FORMAT_VERSION:
        raise OSError(f"{path} implements format {lib.msq_format_version()}, expected {FORMAT_VERSION}")
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MsqError(status, where)


def _host(a, dtype) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def plan(N: int, K: int, bits, perm_row, perm_col) -> dict:
    """Validate a problem on the host (no GPU needed) and return buffer sizes."""
    lib = load_library()
    b = _host(bits, np.uint8)
    pr = _host(perm_row, np.int32)
    pc = _host(perm_col, np.int32)
    if N > 0 and K > 0 and N % 64 == 0 and K % 128 == 0 and b.size != (N // 64) * (K // 128):
        raise ValueError("bits must have (N/64)*(K/128) entries")
    out = _Sizes()
    _check(lib.msq_plan(N, K, b.ctypes.data, pr.ctypes.data, pc.ctypes.data, ctypes.byref(out)),
           "msq_plan")
    return dict(code_bytes=out.code_bytes, scale_bytes=out.scale_bytes, zero_bytes=out.zero_bytes,
                offset_bytes=out.offset_bytes, blocks_per_bits=list(out.blocks_per_bits),
                mean_bits=out.mean_bits)


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _as_bf16_cuda(a, device):
    torch = _torch()
    if isinstance(a, np.ndarray):
        if a.dtype != np.uint16:
            raise TypeError("numpy inputs must be bf16 bit patterns (uint16)")
        a = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    if a.dtype in (torch.int16, torch.uint16):
        a = a.view(torch.bfloat16)
    if a.dtype != torch.bfloat16:
        raise TypeError(f"expected bf16 data, got {a.dtype}")
    return a.to(device).contiguous()


@dataclass
class PackedWeight:
    """Device buffers of one packed weight (format version 2).  Holds the tensors
    so their memory outlives every call that uses the descriptor."""
    N: int
    K: int
    bits: "object"          # uint8 [N/64][K/128]
    perm_row: "object"      # int32 [N]
    perm_col: "object"      # int32 [K]
    block_offset: "object"  # int32 view of uint32 [N/64][K/128]
    codes: "object"         # uint8 [code_bytes] (256-byte aligned by the allocator)
    scale: "object"         # float32 [N/64][K/128][64]
    zero: "object"          # uint8 [N/64][K/128][64]
    code_bytes: int
    mean_bits: float = 0.0
    tile16_blocks: int = 0

    def descriptor(self) -> _Weight:
        w = _Weight()
        w.N, w.K = self.N, self.K
        w.bits = self.bits.data_ptr()
        w.perm_row = self.perm_row.data_ptr()
        w.perm_col = self.perm_col.data_ptr()
        w.block_offset = self.block_offset.data_ptr()
        w.codes = self.codes.data_ptr() if self.code_bytes > 0 else None
        w.scale = self.scale.data_ptr()
        w.zero = self.zero.data_ptr()
        w.code_bytes = self.code_bytes
        w.tile16_blocks = self.tile16_blocks
        return w

    def to_numpy(self) -> dict:
        return dict(bits=self.bits.cpu().numpy(), perm_row=self.perm_row.cpu().numpy(),
                    perm_col=self.perm_col.cpu().numpy(),
                    block_offset=self.block_offset.cpu().numpy().view(np.uint32),
                    codes=self.codes.cpu().numpy()[: self.code_bytes],
                    scale=self.scale.cpu().numpy(), zero=self.zero.cpu().numpy())

    def clone(self) -> "PackedWeight":
        """Independent copy of every buffer (used to defeat caches in benchmarks)."""
        return PackedWeight(self.N, self.K, self.bits.clone(), self.perm_row.clone(),
                            self.perm_col.clone(), self.block_offset.clone(), self.codes.clone(),
                            self.scale.clone(), self.zero.clone(), self.code_bytes, self.mean_bits,
                            self.tile16_blocks)

    @property
    def packed_bytes(self) -> int:
        """Bytes the decode kernel must read for the weight: codes + scale/zero of live
        blocks + bit map and offsets + permutations."""
        nb = int(self.bits.numel())
        live = int((self.bits != 0).sum().item())
        return self.code_bytes + 320 * live + 5 * nb + 4 * (self.N + self.K)


def allocate_packed(N: int, K: int, bits, perm_row, perm_col, device="cuda") -> PackedWeight:
    """Validate the problem on the host (msq_plan, the one validation) and allocate the
    device buffers of its packed weight; the bit map and permutations are copied in."""
    torch = _torch()
    bh = _host(bits, np.uint8)
    if N % 64 == 0 and K % 128 == 0 and N > 0 and K > 0:
        bh = bh.reshape(N // 64, K // 128)
    ph = _host(perm_row, np.int32)
    qh = _host(perm_col, np.int32)
    sizes = plan(N, K, bh, ph, qh)
    dev = torch.device(device)
    code_bytes = int(sizes["code_bytes"])
    return PackedWeight(
        N, K,
        bits=torch.from_numpy(bh.copy()).to(dev),
        perm_row=torch.from_numpy(ph.copy()).to(dev),
        perm_col=torch.from_numpy(qh.copy()).to(dev),
        block_offset=torch.empty(bh.shape, dtype=torch.int32, device=dev),
        codes=torch.empty(max(code_bytes, 256), dtype=torch.uint8, device=dev),
        scale=torch.empty((N // 64, K // 128, 64), dtype=torch.float32, device=dev),
        zero=torch.empty((N // 64, K // 128, 64), dtype=torch.uint8, device=dev),
        code_bytes=code_bytes, mean_bits=float(sizes["mean_bits"]),
        tile16_blocks=int(sizes["blocks_per_bits"][16]))


def pack_into(W, pw: PackedWeight, stream=None) -> PackedWeight:
    """msq_quantize_pack of W (bf16 [N][K] on the weight's device) into the buffers of
    pw (from allocate_packed); asynchronous on the stream."""
    lib = load_library()
    Wd = _as_bf16_cuda(W, pw.bits.device)
    if tuple(Wd.shape) != (pw.N, pw.K):
        raise ValueError(f"W must be [{pw.N}][{pw.K}]")
    w = pw.descriptor()
    _check(lib.msq_quantize_pack(Wd.data_ptr(), ctypes.byref(w), _stream_handle(stream)),
           "msq_quantize_pack")
    return pw


def quantize_pack(W, bits, perm_row, perm_col, device="cuda", stream=None) -> PackedWeight:
    """Quantize and pack W (bf16 [N][K], original order) on the GPU."""
    Wd = _as_bf16_cuda(W, device)
    N, K = int(Wd.shape[0]), int(Wd.shape[1])
    pw = allocate_packed(N, K, bits, perm_row, perm_col, device=Wd.device)
    return pack_into(Wd, pw, stream=stream)


def pack_bytes(pw: PackedWeight) -> int:
    """HBM bytes the pack must move: W read (2 N K), permutations and bit map read,
    offsets, codes, scales and zero points written."""
    nb = int(pw.bits.numel())
    return (2 * pw.N * pw.K + 4 * (pw.N + pw.K) + nb + 4 * nb + pw.code_bytes
            + 4 * pw.N * (pw.K // 128) + pw.N * (pw.K // 128))


def workspace_bytes(M: int, N: int, K: int, kernel: str = "auto",
                    options: Optional[dict] = None) -> int:
    """Workspace of msq_gemm (automatic choices) or of msq_gemm_ex with these choices."""
    o = _options(kernel, options)
    lib = load_library()
    if o is None:
        return int(lib.msq_gemm_workspace_bytes(M, N, K))
    return int(lib.msq_gemm_workspace_bytes_ex(M, N, K, ctypes.byref(o)))


GROUP_MAX = 8


def _descriptor_array(pws):
    descs = [pw.descriptor() for pw in pws]
    arr = (ctypes.POINTER(_Weight) * len(descs))(*[ctypes.pointer(d) for d in descs])
    return descs, arr


def group_workspace_bytes(M: int, pws, options: Optional[dict] = None) -> int:
    descs, arr = _descriptor_array(pws)
    o = _options("auto", options)
    lib = load_library()
    if o is None:
        return int(lib.msq_gemm_group_workspace_bytes(M, arr, len(descs)))
    return int(lib.msq_gemm_group_workspace_bytes_ex(M, arr, len(descs), ctypes.byref(o)))


def gemm_group(xs, pws, outs=None, workspace=None, stream=None, options: Optional[dict] = None):
    """[x_i . W_i^T] for up to GROUP_MAX packed weights in one call (M == 1: one decode
    launch for all of them, plus one prep launch if some have several K ranges; M = 2..32:
    one gather and one decode launch; large M: one gather and one GEMM launch).  xs: one activation per weight (the same tensor may repeat); returns
    the list of fp32 [M][N_i] outputs."""
    torch = _torch()
    lib = load_library()
    pws = list(pws)
    if not 1 <= len(pws) <= GROUP_MAX or len(xs) != len(pws):
        raise ValueError(f"1 to {GROUP_MAX} weights, one activation each")
    xds = [_as_bf16_cuda(x, pw.bits.device) for x, pw in zip(xs, pws)]
    M = int(xds[0].shape[0])
    for xd, pw in zip(xds, pws):
        if xd.dim() != 2 or xd.shape[1] != pw.K or int(xd.shape[0]) != M:
            raise ValueError(f"each x must be [M][K] of its weight, one M for all")
    if outs is None:
        outs = [torch.empty((M, pw.N), dtype=torch.float32, device=xds[0].device) for pw in pws]
    descs, arr = _descriptor_array(pws)
    need = group_workspace_bytes(M, pws, options)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xds[0].device)
    xa = (ctypes.c_void_p * len(xds))(*[xd.data_ptr() for xd in xds])
    ya = (ctypes.c_void_p * len(outs))(*[y.data_ptr() for y in outs])
    o = _options("auto", options)
    if M > 0:
        ws_ptr = workspace.data_ptr() if need > 0 else None
        if o is None:
            st = lib.msq_gemm_group(xa, M, arr, ya, len(descs), ws_ptr, workspace.numel(),
                                    _stream_handle(stream))
        else:
            st = lib.msq_gemm_group_ex(xa, M, arr, ya, len(descs), ws_ptr, workspace.numel(),
                                       ctypes.byref(o), _stream_handle(stream))
        _check(st, "msq_gemm_group")
    return outs


def gemm(x, pw: PackedWeight, kernel: str = "auto", out=None, workspace=None, stream=None,
         options: Optional[dict] = None):
    """y = x . W^T (fp32 [M][N], original row order) from packed weights.  kernel and
    options (keys gemv_split, gemv_waves, m1_prep, gemm_split) select the launch
    (msq_gemm_ex); the defaults are msq_gemm's automatic choices."""
    torch = _torch()
    lib = load_library()
    xd = _as_bf16_cuda(x, pw.bits.device)
    if xd.dim() != 2 or xd.shape[1] != pw.K:
        raise ValueError(f"x must be [M][{pw.K}]")
    M = int(xd.shape[0])
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=xd.device)
    need = workspace_bytes(M, pw.N, pw.K, kernel, options)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xd.device)
    w = pw.descriptor()
    ws_ptr = workspace.data_ptr() if need > 0 else None
    o = _options(kernel, options)
    xp = xd.data_ptr() if M > 0 else None
    yp = out.data_ptr() if M > 0 else None
    if o is None:
        st = lib.msq_gemm(xp, M, ctypes.byref(w), yp, ws_ptr, workspace.numel(),
                          _stream_handle(stream))
    else:
        st = lib.msq_gemm_ex(xp, M, ctypes.byref(w), yp, ws_ptr, workspace.numel(),
                             ctypes.byref(o), _stream_handle(stream))
    _check(st, "msq_gemm")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def gemm_noalloc(x, pw: PackedWeight, out=None, stream=None):
    """msq_gemm_noalloc: y = x . W^T with the library's own static device scratch as the
    workspace (no device allocation inside the call; out is allocated here if None)."""
    torch = _torch()
    lib = load_library()
    xd = _as_bf16_cuda(x, pw.bits.device)
    if xd.dim() != 2 or xd.shape[1] != pw.K:
        raise ValueError(f"x must be [M][{pw.K}]")
    M = int(xd.shape[0])
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=xd.device)
    w = pw.descriptor()
    _check(lib.msq_gemm_noalloc(xd.data_ptr() if M > 0 else None, M, ctypes.byref(w),
                                out.data_ptr() if M > 0 else None, _stream_handle(stream)),
           "msq_gemm_noalloc")
    return out


ALLOC_LEVELS = (0, 1, 2, 3, 4, 8)


def alloc_workspace_bytes(n_blocks: int) -> int:
    return int(load_library().msq_alloc_workspace_bytes(int(n_blocks)))


def allocate_bits(utility, budget_bits: int, workspace=None, stream=None):
    """Bitwidth per block under a budget (msq_allocate_bits).  utility: fp32
    [n_blocks][6] for bitwidths ALLOC_LEVELS (numpy or torch).  Returns (bits as a
    uint8 device tensor [n_blocks], batched iterations)."""
    torch = _torch()
    lib = load_library()
    u = torch.as_tensor(utility)
    if u.dtype != torch.float32 or u.dim() != 2 or u.shape[1] != len(ALLOC_LEVELS):
        raise ValueError("utility must be float32 [n_blocks][6]")
    u = u.to("cuda").contiguous()
    n = int(u.shape[0])
    bits = torch.empty(n, dtype=torch.uint8, device=u.device)
    need = alloc_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=u.device)
    iters = ctypes.c_int32(0)
    _check(lib.msq_allocate_bits(u.data_ptr(), n, int(budget_bits), bits.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), ctypes.byref(iters),
                                 _stream_handle(stream)), "msq_allocate_bits")
    return bits, int(iters.value)


def reorder_channels(saliency, reorder_rows: bool = True, workspace=None, stream=None):
    """(perm_row, perm_col) as int32 device tensors from a saliency map fp32 [N][K]
    (msq_reorder_channels): rows and columns by total saliency, descending."""
    torch = _torch()
    lib = load_library()
    S = torch.as_tensor(saliency)
    if S.dtype != torch.float32 or S.dim() != 2:
        raise ValueError("saliency must be float32 [N][K]")
    S = S.to("cuda").contiguous()
    N, K = int(S.shape[0]), int(S.shape[1])
    pr = torch.empty(N, dtype=torch.int32, device=S.device)
    pc = torch.empty(K, dtype=torch.int32, device=S.device)
    need = int(lib.msq_reorder_workspace_bytes(N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=S.device)
    _check(lib.msq_reorder_channels(S.data_ptr(), N, K, int(bool(reorder_rows)), pr.data_ptr(),
                                    pc.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                    _stream_handle(stream)), "msq_reorder_channels")
    return pr, pc
