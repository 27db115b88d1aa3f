"""MI355X-native NVFP4 weight-only projection GEMV for batched LLM decode.

The compute lives in the HIP library ``libnvfp4.so`` (sources in ``csrc/``,
C ABI in ``include/nvfp4.h``); this module only checks torch tensors and passes
their device pointers and the current HIP stream through ctypes.  Nothing here
computes on the CPU, and every entry point raises if the library is missing.

    W  = torch.randn(N, K, device="cuda") * 0.02
    pw = PackedWeight.from_float(W)            # quantise + pack, once
    Y  = gemv(pw, X)                           # X: bf16 [n, K], n <= 16
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "nvfp4.h")
MAX_TOKENS = 16

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_RANGE", 3: "NVFP4_ERR_ALIGN",
          4: "NVFP4_ERR_SHAPE", 5: "NVFP4_ERR_SCHEDULE", 6: "NVFP4_ERR_LAUNCH",
          7: "NVFP4_ERR_DEVICE", 8: "NVFP4_ERR_WORKSPACE", 9: "NVFP4_ERR_SCRATCH"}


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, strerror(status), STATUS.get(status, status)))


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnvfp4.so is not built (run `python -m nvfp4_weight_only_02_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_packed_codes_bytes.restype = ctypes.c_size_t
        L.nvfp4_packed_codes_bytes.argtypes = [_i32, _i32]
        L.nvfp4_packed_scales_bytes.restype = ctypes.c_size_t
        L.nvfp4_packed_scales_bytes.argtypes = [_i32, _i32]
        L.nvfp4_quantize.restype = _i32
        L.nvfp4_quantize.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp]
        L.nvfp4_quantize_packed.restype = _i32
        L.nvfp4_quantize_packed.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
        L.nvfp4_pack.restype = _i32
        L.nvfp4_pack.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _vp]
        L.nvfp4_gemv.restype = _i32
        L.nvfp4_gemv.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _vp]
        L.nvfp4_gemv_ws.restype = _i32
        L.nvfp4_gemv_ws.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _vp, ctypes.c_size_t, _vp]
        L.nvfp4_gemv_ws_static.restype = _i32
        L.nvfp4_gemv_ws_static.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
        L.nvfp4_gemv_static_scratch_bytes.restype = ctypes.c_size_t
        L.nvfp4_gemv_static_scratch_bytes.argtypes = []
        L.nvfp4_gemv_kparts.restype = _i32
        L.nvfp4_gemv_kparts.argtypes = [_i32, _i32]
        L.nvfp4_gemv_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_gemv_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
        L.nvfp4_gemv_qkv.restype = _i32
        L.nvfp4_gemv_qkv.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                                     _i64, _vp]
        L.nvfp4_gemv_sched.restype = _i32
        L.nvfp4_gemv_sched.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32,
                                       ctypes.POINTER(ctypes.c_uint8), _i32, _vp]
        L.nvfp4_schedule.restype = _i32
        L.nvfp4_schedule.argtypes = [_i32, _i32, _i32, ctypes.POINTER(ctypes.c_uint8), _i32]
        L.nvfp4_schedule_greedy.restype = _i32
        L.nvfp4_schedule_greedy.argtypes = [_i32, _i32, ctypes.POINTER(ctypes.c_uint8), _i32]
        L.nvfp4_launch_geometry.restype = _i32
        L.nvfp4_launch_geometry.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_i32),
                                            ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
        L.nvfp4_gemv_variant.restype = _i32
        L.nvfp4_gemv_variant.argtypes = [_i32, _i32, _i32, _i32, ctypes.POINTER(_i32)]
        L.nvfp4_gemm.restype = _i32
        L.nvfp4_gemm.argtypes = [_vp, _vp, ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _vp]
        L.nvfp4_gemm_geometry.restype = _i32
        L.nvfp4_gemm_geometry.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                          ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
        L.nvfp4_strerror.restype = ctypes.c_char_p
        L.nvfp4_strerror.argtypes = [_i32]
        _lib = L
    return _lib


def header_functions(path: str = HEADER_PATH) -> list:
    """Names of the functions a header under include/ declares (nvfp4.h by default)."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nvfp4_\w+)\s*\(", text, re.M)))


def strerror(status: int) -> str:
    return lib().nvfp4_strerror(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Nvfp4Error(status, what)


def check_devices(devices, current: int, stream_device) -> None:
    """The library launches on the current device, on the given stream: every
    tensor of a call and the stream must be on that device.  Raises ValueError
    naming the mismatch (a pure function of torch.device values)."""
    want = torch.device("cuda", current)
    for d in devices:
        if d != want:
            raise ValueError("a tensor is on %s but the library launches on the current device %s "
                             "(select it with torch.cuda.device)" % (d, want))
    if stream_device != want:
        raise ValueError("the stream is on %s but the library launches on the current device %s"
                         % (stream_device, want))


def _stream(stream, *tensors):
    """The HIP stream of a launch (the current stream unless one is given),
    after checking that it and every tensor are on the current device."""
    s = stream if stream is not None else torch.cuda.current_stream()
    check_devices([t.device for t in tensors], torch.cuda.current_device(), s.device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


# ---- sizes, schedules, geometry (host-only) -------------------------------

def packed_codes_bytes(N: int, K: int) -> int:
    return int(lib().nvfp4_packed_codes_bytes(N, K))


def packed_scales_bytes(N: int, K: int) -> int:
    return int(lib().nvfp4_packed_scales_bytes(N, K))


def schedule(n: int, N: int, K: int) -> list:
    buf = (ctypes.c_uint8 * MAX_TOKENS)()
    cnt = lib().nvfp4_schedule(n, N, K, buf, MAX_TOKENS)
    if cnt < 0:
        raise Nvfp4Error(-cnt, "nvfp4_schedule")
    return list(buf[:cnt])


def schedule_greedy(n: int, width: int = 3) -> list:
    buf = (ctypes.c_uint8 * MAX_TOKENS)()
    cnt = lib().nvfp4_schedule_greedy(n, width, buf, MAX_TOKENS)
    if cnt < 0:
        raise Nvfp4Error(-cnt, "nvfp4_schedule_greedy")
    return list(buf[:cnt])


def launch_geometry(n: int, N: int, K: int):
    wg, wv, tpw = _i32(), _i32(), _i32()
    _check(lib().nvfp4_launch_geometry(n, N, K, ctypes.byref(wg), ctypes.byref(wv),
                                       ctypes.byref(tpw)), "nvfp4_launch_geometry")
    return wg.value, wv.value, tpw.value


def gemv_variant(n: int, N: int, K: int, ks: int = 1) -> tuple:
    """(tiles per wave, token groups of four, exact, K-chunk passes, K parts)
    of the GEMV kernel a call launches; ks = 1 for nvfp4_gemv, 0 for
    nvfp4_gemv_ws's own part count, > 1 for that many parts."""
    v = (_i32 * 5)()
    _check(lib().nvfp4_gemv_variant(n, N, K, ks, v), "nvfp4_gemv_variant")
    return tuple(v)


def gemm_geometry(n: int, N: int, K: int):
    """(rows per workgroup, tokens per workgroup, grid_x, grid_y) of nvfp4_gemm."""
    r, t, gx, gy = _i32(), _i32(), _i32(), _i32()
    _check(lib().nvfp4_gemm_geometry(n, N, K, ctypes.byref(r), ctypes.byref(t), ctypes.byref(gx),
                                     ctypes.byref(gy)), "nvfp4_gemm_geometry")
    return r.value, t.value, gx.value, gy.value


# ---- weight preparation ----------------------------------------------------

def quantize(W: torch.Tensor, stream=None):
    """fp32 [N, K] (device) -> canonical (codes u8 [N, K/2], scales u8 [N, K/16],
    tensor_scale f32[2] = [gscale, amax]), all on the device."""
    _dev(W, torch.float32, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((N, max(K // 16, 1)), dtype=torch.uint8, device=W.device)
    ts = torch.empty(2, dtype=torch.float32, device=W.device)
    _check(lib().nvfp4_quantize(W.data_ptr(), N, K, codes.data_ptr(), scales.data_ptr(),
                                ts.data_ptr(), _stream(stream, W)), "nvfp4_quantize")
    return codes, scales, ts


def quantize_packed(W: torch.Tensor, stream=None):
    """fp32 or bf16 [N, K] (device) -> packed device layout directly
    (codes, scales, tensor_scale f32[2] = [gscale, amax]), all on the device."""
    if not isinstance(W, torch.Tensor) or W.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("W must be a float32 or bfloat16 tensor")
    _dev(W, W.dtype, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    cp = torch.empty(packed_codes_bytes(N, K), dtype=torch.uint8, device=W.device)
    sp = torch.empty(packed_scales_bytes(N, K), dtype=torch.uint8, device=W.device)
    ts = torch.empty(2, dtype=torch.float32, device=W.device)
    dtype = 0 if W.dtype == torch.float32 else 1
    _check(lib().nvfp4_quantize_packed(W.data_ptr(), dtype, N, K, cp.data_ptr(), sp.data_ptr(),
                                       ts.data_ptr(), _stream(stream, W)), "nvfp4_quantize_packed")
    return cp, sp, ts


def pack(codes: torch.Tensor, scales: torch.Tensor, N: int, K: int, stream=None):
    """Canonical codes/scales (device) -> packed device layout."""
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales")
    if codes.numel() != N * (K // 2) or scales.numel() != N * (K // 16):
        raise ValueError("codes/scales do not match N x K")
    cp = torch.empty(packed_codes_bytes(N, K), dtype=torch.uint8, device=codes.device)
    sp = torch.empty(packed_scales_bytes(N, K), dtype=torch.uint8, device=codes.device)
    _check(lib().nvfp4_pack(codes.data_ptr(), scales.data_ptr(), N, K, cp.data_ptr(),
                            sp.data_ptr(), _stream(stream, codes, scales)), "nvfp4_pack")
    return cp, sp


@dataclass
class PackedWeight:
    """An NVFP4 weight in the packed device layout."""
    codes: torch.Tensor      # u8, packed_codes_bytes(N, K)
    scales: torch.Tensor     # u8, packed_scales_bytes(N, K)
    gscale: float
    N: int
    K: int

    @classmethod
    def from_canonical(cls, codes: torch.Tensor, scales: torch.Tensor, gscale: float,
                       N: int, K: int, stream=None) -> "PackedWeight":
        cp, sp = pack(codes, scales, N, K, stream)
        return cls(cp, sp, float(gscale), N, K)

    @classmethod
    def from_float(cls, W: torch.Tensor, stream=None) -> "PackedWeight":
        """Quantise an fp32 or bf16 weight straight into the packed layout."""
        cp, sp, ts = quantize_packed(W, stream)
        gscale = float(ts[0].item())          # one host read at load time
        return cls(cp, sp, gscale, W.shape[0], W.shape[1])


# ---- the GEMV --------------------------------------------------------------

def _x(X: torch.Tensor, K: int) -> torch.Tensor:
    _dev(X, torch.bfloat16, "X")
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [n, %d]" % K)
    return X


def gemv(w: PackedWeight, X: torch.Tensor, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Y[n, N] = X[n, K] . dequant(W)^T (bf16 in and out, fp32 accumulation)."""
    _x(X, w.K)
    n = X.shape[0]
    Y = out if out is not None else torch.empty((n, w.N), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.shape != (n, w.N):
        raise ValueError("out must be [n, N]")
    _check(lib().nvfp4_gemv(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                            Y.data_ptr(), n, w.N, w.K, _stream(stream, w.codes, w.scales, X, Y)), "nvfp4_gemv")
    return Y


def gemv_kparts(N: int, K: int) -> int:
    """K parts gemv_ws takes by default for an N x K weight."""
    ks = lib().nvfp4_gemv_kparts(N, K)
    if ks < 0:
        raise Nvfp4Error(-ks, "nvfp4_gemv_kparts")
    return ks


def gemv_workspace_bytes(n: int, N: int, K: int, ks: int = 0) -> int:
    """Workspace bytes gemv_ws needs (0 when it needs none)."""
    return int(lib().nvfp4_gemv_workspace_bytes(n, N, K, ks))


def gemv_ws(w: PackedWeight, X: torch.Tensor, ks: int = 0, workspace: torch.Tensor = None,
            out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """gemv with K cut into ``ks`` parts (0: the library's choice for the
    shape): fp32 partials in ``workspace`` (a uint8 device tensor, allocated
    here when not given), then a fixed-order sum of the parts."""
    _x(X, w.K)
    n = X.shape[0]
    Y = out if out is not None else torch.empty((n, w.N), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.shape != (n, w.N):
        raise ValueError("out must be [n, N]")
    if workspace is None:
        need = gemv_workspace_bytes(n, w.N, w.K, ks)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device)
    _dev(workspace, torch.uint8, "workspace")
    _check(lib().nvfp4_gemv_ws(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                               Y.data_ptr(), n, w.N, w.K, int(ks), workspace.data_ptr(),
                               workspace.numel(), _stream(stream, w.codes, w.scales, X, Y, workspace)),
           "nvfp4_gemv_ws")
    return Y


def gemv_ws_static(w: PackedWeight, X: torch.Tensor, ks: int = 0, out: torch.Tensor = None,
                   stream=None) -> torch.Tensor:
    """gemv_ws with the partials in the library's fixed scratch memory: no
    device allocation by the library (``out`` may be given to avoid torch's).
    Calls that overlap on one GPU race."""
    _x(X, w.K)
    n = X.shape[0]
    Y = out if out is not None else torch.empty((n, w.N), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.shape != (n, w.N):
        raise ValueError("out must be [n, N]")
    _check(lib().nvfp4_gemv_ws_static(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                                      Y.data_ptr(), n, w.N, w.K, int(ks),
                                      _stream(stream, w.codes, w.scales, X, Y)),
           "nvfp4_gemv_ws_static")
    return Y


def gemv_static_scratch_bytes() -> int:
    return int(lib().nvfp4_gemv_static_scratch_bytes())


def gemv_sched(w: PackedWeight, X: torch.Tensor, tile_widths, out: torch.Tensor = None,
               stream=None) -> torch.Tensor:
    """gemv with an explicit token-tile schedule (one weight read per tile)."""
    _x(X, w.K)
    n = X.shape[0]
    Y = out if out is not None else torch.empty((n, w.N), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.shape != (n, w.N):
        raise ValueError("out must be [n, N]")
    widths = (ctypes.c_uint8 * max(len(tile_widths), 1))(*[int(v) for v in tile_widths])
    _check(lib().nvfp4_gemv_sched(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                                  Y.data_ptr(), n, w.N, w.K, widths, len(tile_widths),
                                  _stream(stream, w.codes, w.scales, X, Y)), "nvfp4_gemv_sched")
    return Y


def gemm(w: PackedWeight, X: torch.Tensor, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Prefill form: Y[n, N] = X[n, K] . dequant(W)^T for any n >= 1 (tiled
    MFMA GEMM; bf16 in and out, fp32 accumulation)."""
    _x(X, w.K)
    n = X.shape[0]
    Y = out if out is not None else torch.empty((n, w.N), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.shape != (n, w.N):
        raise ValueError("out must be [n, N]")
    _check(lib().nvfp4_gemm(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                            Y.data_ptr(), n, w.N, w.K, _stream(stream, w.codes, w.scales, X, Y)), "nvfp4_gemm")
    return Y


def gemv_qkv(w: PackedWeight, X: torch.Tensor, rows, out_off, ldy: int,
             out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Fused q|k|v projection writing each projection at its offset of a
    token-major output with ``ldy`` elements per token."""
    _x(X, w.K)
    n = X.shape[0]
    if len(rows) != 3 or len(out_off) != 3:
        raise ValueError("rows and out_off take three entries (q, k, v)")
    if sum(rows) != w.N:
        raise ValueError("rows must sum to N")
    Y = out if out is not None else torch.empty((n, ldy), dtype=torch.bfloat16, device=X.device)
    _dev(Y, torch.bfloat16, "out")
    if Y.numel() < n * ldy:
        raise ValueError("out is smaller than n * ldy")
    r = (ctypes.c_int32 * 3)(*[int(v) for v in rows])
    o = (ctypes.c_int64 * 3)(*[int(v) for v in out_off])
    _check(lib().nvfp4_gemv_qkv(w.codes.data_ptr(), w.scales.data_ptr(), w.gscale, X.data_ptr(),
                                Y.data_ptr(), n, w.K, r, o, int(ldy),
                                _stream(stream, w.codes, w.scales, X, Y)),
           "nvfp4_gemv_qkv")
    return Y
