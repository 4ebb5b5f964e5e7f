"""Python binding of libsvq (include/svq.h): weight-only quantized linear layers
(W4A16 GPTQ-style INT4, MXFP8) for decode and speculative-verify shapes on
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libsvq.so, which must be built in-tree (``python -m
spec_verify_amd.build``). There is no CPU or PyTorch fallback: if the library
is missing or a call fails, an exception is raised.

PyTorch supplies device memory and the current stream; tensors are passed as
raw device pointers. bf16/fp16 values travel as torch.bfloat16/float16 tensors
or as their 16-bit patterns in int16/uint16 tensors.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "SvqError", "KERNEL_AUTO", "KERNEL_DOT2", "KERNEL_MFMA_SKINNY", "KERNEL_MFMA_WIDE",
    "lib", "library_path", "q4_repack", "w4a16_gemm", "mxfp8_gemm", "w4a16_kernel_name",
    "mxfp8_kernel_name", "w4a16_workspace_bytes", "mxfp8_workspace_bytes", "Workspace",
    "EXPORTED_SYMBOLS", "rtn_quantize", "w8a16_gemm", "w8a16_workspace_bytes", "w8a16_kernel_name",
    "fuse_projections", "fuse_or_keep", "ct_to_gptq", "MAX_FUSED_PARTS", "mxfp8_quantize",
    "OP_W4A16", "OP_MXFP8", "OP_W8A16", "workspace_bytes", "kernel_name",
    "launch_geometry", "stream_probe",
]

KERNEL_AUTO, KERNEL_DOT2, KERNEL_MFMA_SKINNY, KERNEL_MFMA_WIDE = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libsvq.so")

EXPORTED_SYMBOLS = (
    "svq_abi_version", "svq_status_string", "svq_q4_repacked_bytes", "svq_q4_repack",
    "svq_w4a16_workspace_bytes", "svq_w4a16_gemm", "svq_w4a16_gemm_with",
    "svq_w4a16_kernel_name", "svq_mxfp8_workspace_bytes", "svq_mxfp8_gemm",
    "svq_mxfp8_gemm_with", "svq_mxfp8_kernel_name", "svq_rtn_quantize",
    "svq_w8a16_workspace_bytes", "svq_w8a16_gemm", "svq_w8a16_kernel_name",
    "svq_fuse_projections", "svq_ct_to_gptq", "svq_mxfp8_quantize", "svq_workspace_bytes",
    "svq_kernel_name", "svq_launch_geometry", "svq_stream_probe", "svq_mfma_probe", "svq_mxfp8_repack",
    "svq_w4a16_gemm_noalloc",
)

OP_W4A16, OP_MXFP8, OP_W8A16 = 1, 2, 3

MAX_FUSED_PARTS = 16

_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_lib = None
_lock = threading.Lock()


class SvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: svq status {status}: {_status_text(status)}")


def lib():
    """The loaded libsvq.so (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"libsvq.so not found at {library_path}; build it with "
                "`python -m spec_verify_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(library_path)
        L.svq_abi_version.restype = ctypes.c_int
        L.svq_status_string.restype = ctypes.c_char_p
        L.svq_status_string.argtypes = [ctypes.c_int]
        L.svq_q4_repacked_bytes.restype = _sz
        L.svq_q4_repacked_bytes.argtypes = [_i64, _i64]
        L.svq_q4_repack.restype = ctypes.c_int
        L.svq_q4_repack.argtypes = [_p, _p, _i64, _i64, _p]
        L.svq_w4a16_workspace_bytes.restype = _sz
        L.svq_w4a16_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i32]
        L.svq_w4a16_gemm.restype = ctypes.c_int
        L.svq_w4a16_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.svq_w4a16_gemm_with.restype = ctypes.c_int
        L.svq_w4a16_gemm_with.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.svq_w4a16_kernel_name.restype = ctypes.c_char_p
        L.svq_w4a16_kernel_name.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i32]
        L.svq_mxfp8_workspace_bytes.restype = _sz
        L.svq_mxfp8_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i64]
        L.svq_mxfp8_gemm.restype = ctypes.c_int
        L.svq_mxfp8_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.svq_mxfp8_gemm_with.restype = ctypes.c_int
        L.svq_mxfp8_gemm_with.argtypes = [ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.svq_mxfp8_kernel_name.restype = ctypes.c_char_p
        L.svq_mxfp8_kernel_name.argtypes = [ctypes.c_int, _i64, _i64, _i64]
        L.svq_rtn_quantize.restype = ctypes.c_int
        L.svq_rtn_quantize.argtypes = [_p, _i32, _i32, _p, _p, _i64, _i64, _p]
        L.svq_w8a16_workspace_bytes.restype = _sz
        L.svq_w8a16_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32]
        L.svq_w8a16_gemm.restype = ctypes.c_int
        L.svq_w8a16_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.svq_w8a16_kernel_name.restype = ctypes.c_char_p
        L.svq_w8a16_kernel_name.argtypes = [_i64, _i64, _i64, _i32]
        L.svq_fuse_projections.restype = ctypes.c_int
        L.svq_fuse_projections.argtypes = [_i32, _p, _p, _p, _i32, _i64, _i32, _p, _p, _p]
        L.svq_ct_to_gptq.restype = ctypes.c_int
        L.svq_mxfp8_quantize.restype = ctypes.c_int
        L.svq_mxfp8_quantize.argtypes = [_p, _i32, _p, _p, _i64, _i64, _p]
        L.svq_ct_to_gptq.argtypes = [_p, _p, _p, _p, _i64, _i64, _i32, _p]
        L.svq_workspace_bytes.restype = _sz
        L.svq_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i32]
        L.svq_kernel_name.restype = ctypes.c_char_p
        L.svq_kernel_name.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i32]
        L.svq_launch_geometry.restype = ctypes.c_int
        L.svq_launch_geometry.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _i32,
                                          ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.POINTER(_sz)]
        L.svq_stream_probe.restype = ctypes.c_int
        L.svq_stream_probe.argtypes = [_p, _sz, ctypes.c_uint32, ctypes.c_uint32, _p, _p]
        L.svq_mxfp8_repack.restype = ctypes.c_int
        L.svq_mxfp8_repack.argtypes = [_p, _p, _i64, _i64, _p]
        L.svq_mfma_probe.restype = ctypes.c_int
        L.svq_mfma_probe.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, _i32, _p, _p]
        L.svq_w4a16_gemm_noalloc.restype = ctypes.c_int
        L.svq_w4a16_gemm_noalloc.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p]
        _lib = L
        return L


def _status_text(status: int) -> str:
    try:
        return lib().svq_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - library missing
        return "unknown"


def _check(status: int, where: str) -> None:
    if status != 0:
        raise SvqError(status, where)


# ---- torch plumbing ------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev_ptr(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check_elem(t, name, bytes_per_elem):
    if t.element_size() != bytes_per_elem:
        raise TypeError(f"{name} must have {bytes_per_elem}-byte elements, got {t.dtype}")


class Workspace:
    """Zero-filled device scratch for the split-K arrival counters and partials.

    One per (device, stream); grows on demand (a new buffer is zero-filled). The
    kernels leave the counters at zero after every call, so the buffer can be
    reused by later calls on the same stream without clearing it again.
    """

    _cache: dict = {}

    @classmethod
    def get(cls, nbytes: int, device, stream_handle: int):
        torch = _torch()
        if nbytes == 0:
            return None
        key = (device.index, stream_handle)
        buf = cls._cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            cls._cache[key] = buf
        return buf


def w4a16_workspace_bytes(M, N, K, group_size=128, kernel=KERNEL_AUTO) -> int:
    v = lib().svq_w4a16_workspace_bytes(kernel, M, N, K, group_size)
    if v == ctypes.c_size_t(-1).value:
        raise SvqError(10, "svq_w4a16_workspace_bytes")
    return v


def mxfp8_workspace_bytes(M, N, K, kernel=KERNEL_AUTO) -> int:
    v = lib().svq_mxfp8_workspace_bytes(kernel, M, N, K)
    if v == ctypes.c_size_t(-1).value:
        raise SvqError(10, "svq_mxfp8_workspace_bytes")
    return v


def w4a16_kernel_name(M, N, K, group_size=128, kernel=KERNEL_AUTO):
    r = lib().svq_w4a16_kernel_name(kernel, M, N, K, group_size)
    return r.decode() if r else None


def mxfp8_kernel_name(M, N, K, kernel=KERNEL_AUTO):
    r = lib().svq_mxfp8_kernel_name(kernel, M, N, K)
    return r.decode() if r else None


def workspace_bytes(op, M, N, K, group_size=128) -> int:
    """Workspace bytes of the GEMM of `op` (OP_W4A16, OP_MXFP8 with group_size 32,
    OP_W8A16) with its automatic kernel choice."""
    v = lib().svq_workspace_bytes(op, M, N, K, group_size)
    if v == ctypes.c_size_t(-1).value:
        raise SvqError(10, "svq_workspace_bytes")
    return v


def kernel_name(op, M, N, K, group_size=128):
    """Name of the kernel the GEMM of `op` would launch, or None."""
    r = lib().svq_kernel_name(op, M, N, K, group_size)
    return r.decode() if r else None


def launch_geometry(op, M, N, K, group_size=128, kernel=KERNEL_AUTO):
    """(grid, threads, dynamic LDS bytes) the GEMM call would launch with."""
    g, t, l = ctypes.c_uint64(), ctypes.c_uint32(), _sz()
    _check(lib().svq_launch_geometry(op, kernel, M, N, K, group_size, ctypes.byref(g), ctypes.byref(t),
                                     ctypes.byref(l)), "svq_launch_geometry")
    return g.value, t.value, l.value


def stream_probe(src, nbytes, grid, threads, sink):
    """Read-only stream of the first nbytes of the device tensor src in (grid,
    threads); sink is a device tensor of at least grid 32-bit words."""
    if nbytes > src.numel() * src.element_size() or sink.numel() * sink.element_size() < 4 * grid:
        raise ValueError("src or sink too small")
    _check(lib().svq_stream_probe(_dev_ptr(src, "src"), nbytes, grid, threads, _dev_ptr(sink, "sink"),
                                  _stream_ptr(src)), "svq_stream_probe")


def mfma_probe(grid, threads, per_wave, sink, random_operands=False):
    """per_wave bf16 16x16x32 MFMAs per wave of (grid, threads), no memory
    traffic; sink is a device tensor of at least grid floats. random_operands
    selects random activation-like A and 128 + q B operands instead of one
    constant value (the chip clocks lower under the switching of real data)."""
    if sink.numel() * sink.element_size() < 4 * grid:
        raise ValueError("sink too small")
    _check(lib().svq_mfma_probe(grid, threads, per_wave, 1 if random_operands else 0, _dev_ptr(sink, "sink"),
                                _stream_ptr(sink)),
           "svq_mfma_probe")


def q4_repack(qweight, out=None):
    """GPTQ int32 [K/8, N] (device) -> tiled int32 buffer of K*N/8 words."""
    torch = _torch()
    K8, N = qweight.shape
    _check_elem(qweight, "qweight", 4)
    if out is None:
        out = torch.empty(K8 * N, dtype=torch.int32, device=qweight.device)
    _check_elem(out, "out", 4)
    if out.numel() * 4 < K8 * N * 4:
        raise ValueError("out too small")
    _check(lib().svq_q4_repack(_dev_ptr(qweight, "qweight"), _dev_ptr(out, "out"), N, K8 * 8,
                               _stream_ptr(qweight)), "svq_q4_repack")
    return out


def w4a16_gemm(x, qweight_tiled, scales, N, group_size=128, out=None, kernel=KERNEL_AUTO,
               workspace=None):
    """bf16 x [M, K] . deq(W)^T -> bf16 [M, N]; W given as the svq_q4_repack output."""
    torch = _torch()
    M, K = x.shape
    _check_elem(x, "x", 2)
    _check_elem(scales, "scales", 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check_elem(out, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    stream = _stream_ptr(x)
    if workspace is None:
        nbytes = w4a16_workspace_bytes(M, N, K, group_size, kernel)
        workspace = Workspace.get(nbytes, x.device, stream.value or 0)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().svq_w4a16_gemm_with(kernel, _dev_ptr(x, "x"), _dev_ptr(qweight_tiled, "qweight_tiled"),
                                     _dev_ptr(scales, "scales"), _dev_ptr(out, "out"), M, N, K,
                                     group_size, ws_ptr, ws_bytes, stream), "svq_w4a16_gemm")
    return out


def mxfp8_repack(w, out=None):
    """E4M3 codes [N, K] (device uint8) -> the tile layout the GEMM reads (flat
    uint8, N*K bytes)."""
    torch = _torch()
    N, K = w.shape
    _check_elem(w, "w", 1)
    if out is None:
        out = torch.empty(N * K, dtype=torch.uint8, device=w.device)
    _check_elem(out, "out", 1)
    if out.numel() < N * K:
        raise ValueError("out too small")
    _check(lib().svq_mxfp8_repack(_dev_ptr(w, "w"), _dev_ptr(out, "out"), N, K, _stream_ptr(w)),
           "svq_mxfp8_repack")
    return out


def mxfp8_gemm(x, w_tiled, scales, out=None, kernel=KERNEL_AUTO, workspace=None):
    """bf16 x [M, K] . (E4M3 w [N, K] * 2^(E8M0 scales [N, K/32] - 127))^T -> bf16 [M, N].

    w_tiled is the flat output of mxfp8_repack; N comes from scales [N, K/32]."""
    torch = _torch()
    M, K = x.shape
    N = scales.shape[0]
    if w_tiled.dim() != 1:
        raise ValueError("w_tiled must be the flat output of mxfp8_repack")
    if w_tiled.numel() != N * K or tuple(scales.shape) != (N, K // 32):
        raise ValueError("w_tiled must hold N*K codes and scales must be [N, K/32]")
    w = w_tiled
    _check_elem(x, "x", 2)
    _check_elem(w, "w", 1)
    _check_elem(scales, "scales", 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check_elem(out, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    stream = _stream_ptr(x)
    if workspace is None:
        nbytes = mxfp8_workspace_bytes(M, N, K, kernel)
        workspace = Workspace.get(nbytes, x.device, stream.value or 0)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().svq_mxfp8_gemm_with(kernel, _dev_ptr(x, "x"), _dev_ptr(w, "w"), _dev_ptr(scales, "scales"),
                                     _dev_ptr(out, "out"), M, N, K, 32, ws_ptr, ws_bytes, stream),
           "svq_mxfp8_gemm")
    return out


def mxfp8_quantize(w, optimized=True, codes=None, scales=None):
    """MXFP8 quantization of bf16 w [N, K] (device): E4M3 codes [N, K] and E8M0
    scales [N, K/32] (uint8), the mxfp8_gemm input. optimized=True keeps, per
    32-element block, the best of the baseline, doubled and halved scale."""
    torch = _torch()
    N, K = w.shape
    _check_elem(w, "w", 2)
    if codes is None:
        codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
    _check_elem(codes, "codes", 1)
    _check_elem(scales, "scales", 1)
    if codes.numel() != N * K or scales.numel() != N * (K // 32):
        raise ValueError("codes or scales have the wrong size")
    _check(lib().svq_mxfp8_quantize(_dev_ptr(w, "w"), 1 if optimized else 0, _dev_ptr(codes, "codes"),
                                    _dev_ptr(scales, "scales"), N, K, _stream_ptr(w)), "svq_mxfp8_quantize")
    return codes, scales


# ---- quantized vocabulary head ----------------------------------------------------

def rtn_quantize(w, bits=8, group_size=128, codes=None, scales=None):
    """Load-time symmetric group-wise RTN of bf16 w [N, K] (device).

    Returns (codes, scales): int8 codes [N, K] for bits=8, GPTQ int32 words
    [K/8, N] (the svq_q4_repack input) for bits=4; fp16 scales [K/G, N].
    """
    torch = _torch()
    N, K = w.shape
    _check_elem(w, "w", 2)
    if codes is None:
        codes = (torch.empty((N, K), dtype=torch.int8, device=w.device) if bits == 8
                 else torch.empty((K // 8, N), dtype=torch.int32, device=w.device))
    if scales is None:
        scales = torch.empty((K // group_size, N), dtype=torch.float16, device=w.device)
    _check_elem(scales, "scales", 2)
    if codes.numel() * codes.element_size() != N * K * bits // 8 or scales.numel() != (K // group_size) * N:
        raise ValueError("codes or scales have the wrong size")
    _check(lib().svq_rtn_quantize(_dev_ptr(w, "w"), bits, group_size, _dev_ptr(codes, "codes"),
                                  _dev_ptr(scales, "scales"), N, K, _stream_ptr(w)), "svq_rtn_quantize")
    return codes, scales


def w8a16_workspace_bytes(M, N, K, group_size=128) -> int:
    v = lib().svq_w8a16_workspace_bytes(M, N, K, group_size)
    if v == ctypes.c_size_t(-1).value:
        raise SvqError(10, "svq_w8a16_workspace_bytes")
    return v


def w8a16_kernel_name(M, N, K, group_size=128):
    r = lib().svq_w8a16_kernel_name(M, N, K, group_size)
    return r.decode() if r else None


def w8a16_gemm(x, w, scales, group_size=128, out=None, workspace=None):
    """bf16 x [M, K] . (int8 w [N, K] * fp16 scales [K/G, N])^T -> bf16 [M, N], M <= 16."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _check_elem(x, "x", 2)
    _check_elem(w, "w", 1)
    _check_elem(scales, "scales", 2)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check_elem(out, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")
    stream = _stream_ptr(x)
    if workspace is None:
        nbytes = w8a16_workspace_bytes(M, N, K, group_size)
        workspace = Workspace.get(nbytes, x.device, stream.value or 0)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().svq_w8a16_gemm(_dev_ptr(x, "x"), _dev_ptr(w, "w"), _dev_ptr(scales, "scales"),
                                _dev_ptr(out, "out"), M, N, K, group_size, ws_ptr, ws_bytes, stream),
           "svq_w8a16_gemm")
    return out


# ---- setup-time projection fusion and compressed-tensors ingest --------------------

def _part_shape(w, s, bits):
    """(K, N) of one quantized projection, from its weights and fp16 scales."""
    if bits == 4:
        _check_elem(w, "weights", 4)
        K, N = w.shape[0] * 8, w.shape[1]
    else:
        _check_elem(w, "weights", 1)
        N, K = w.shape
    _check_elem(s, "scales", 2)
    return K, N


def fuse_projections(parts, bits=4, group_size=128, weight_fused=None, scales_fused=None):
    """Concatenate quantized projections that read the same x along N (device).

    parts: [(weights, scales), ...] with GPTQ int32 words [K/8, N_p] (bits=4)
    or int8 codes [N_p, K] (bits=8) and fp16 scales [K/G, N_p]. Returns
    (weight_fused, scales_fused): the repacked tiles of the fused int4 weight
    (flat int32, ready for w4a16_gemm) or int8 codes [N, K]; fp16 [K/G, N].
    Raises SvqError if the projections cannot be fused.
    """
    torch = _torch()
    if not 1 <= len(parts) <= MAX_FUSED_PARTS:
        raise SvqError(2, "svq_fuse_projections")
    shapes = [_part_shape(w, s, bits) for w, s in parts]
    K = shapes[0][0]
    if any(k != K for k, _ in shapes):
        raise ValueError("projections with different K cannot be fused")
    Nt = sum(n for _, n in shapes)
    dev = parts[0][0].device
    if weight_fused is None:
        weight_fused = (torch.empty(K * Nt // 8, dtype=torch.int32, device=dev) if bits == 4
                        else torch.empty((Nt, K), dtype=torch.int8, device=dev))
    if scales_fused is None:
        scales_fused = torch.empty((K // group_size, Nt), dtype=torch.float16, device=dev)
    if weight_fused.numel() * weight_fused.element_size() != Nt * K * bits // 8 or \
            scales_fused.numel() * scales_fused.element_size() != (K // group_size) * Nt * 2:
        raise ValueError("weight_fused or scales_fused has the wrong size")
    P = len(parts)
    wp = (ctypes.c_void_p * P)(*[_dev_ptr(w, "weights").value for w, _ in parts])
    sp = (ctypes.c_void_p * P)(*[_dev_ptr(s, "scales").value for _, s in parts])
    nn = (ctypes.c_int64 * P)(*[n for _, n in shapes])
    _check(lib().svq_fuse_projections(bits, wp, sp, nn, P, K, group_size,
                                      _dev_ptr(weight_fused, "weight_fused"),
                                      _dev_ptr(scales_fused, "scales_fused"),
                                      _stream_ptr(parts[0][0])), "svq_fuse_projections")
    return weight_fused, scales_fused


def fuse_or_keep(parts, bits=4, group_size=128):
    """fuse_projections, or None with a warning when the projections do not fit.

    Projections that cannot be fused (different K, a width that is not a
    multiple of 16, scales of another group size) keep their own weights: the
    caller then runs one GEMM per projection.
    """
    import warnings
    try:
        return fuse_projections(parts, bits, group_size)
    except (SvqError, ValueError) as e:
        warnings.warn(f"projections not fused, kept separate: {e}", RuntimeWarning, stacklevel=2)
        return None


def ct_to_gptq(weight_packed, weight_scale, group_size=128, qweight=None, scales=None):
    """Compressed-tensors int32 [N, K/8] words and fp16 [N, K/G] scales (device)
    -> GPTQ int32 [K/8, N] and fp16 [K/G, N] (a transpose; no value changes)."""
    torch = _torch()
    N, K8 = weight_packed.shape
    K = K8 * 8
    _check_elem(weight_packed, "weight_packed", 4)
    _check_elem(weight_scale, "weight_scale", 2)
    if tuple(weight_scale.shape) != (N, K // group_size):
        raise ValueError(f"weight_scale must have shape {(N, K // group_size)}")
    if qweight is None:
        qweight = torch.empty((K8, N), dtype=torch.int32, device=weight_packed.device)
    if scales is None:
        scales = torch.empty((K // group_size, N), dtype=torch.float16, device=weight_packed.device)
    _check_elem(qweight, "qweight", 4)
    _check_elem(scales, "scales", 2)
    if qweight.numel() != K8 * N or scales.numel() != (K // group_size) * N:
        raise ValueError("qweight or scales has the wrong size")
    _check(lib().svq_ct_to_gptq(_dev_ptr(weight_packed, "weight_packed"), _dev_ptr(weight_scale, "weight_scale"),
                                _dev_ptr(qweight, "qweight"), _dev_ptr(scales, "scales"), N, K, group_size,
                                _stream_ptr(weight_packed)), "svq_ct_to_gptq")
    return qweight, scales
