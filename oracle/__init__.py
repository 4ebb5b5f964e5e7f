"""CPU oracle for the weight-only quantized linear layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only permitted users. The product package
(spec_verify_amd) never imports this module, and this module never imports the
product package. The arithmetic lives in ``oracle.c`` (plain C, built with gcc,
OpenMP over output columns); every function there writes out the plain
definition of the quantized matmul with k ascending.

The load-time round-to-nearest quantizer of the vocabulary head
(``rtn_quantize``) is written here in numpy, in fp32 arithmetic step by step,
and so are the setup-time layout steps that involve no arithmetic: projection
fusion (``fuse_projections``, concatenation along N) and the compressed-tensors
ingest (``ct_to_gptq``, a transpose of words and scales).

Functions with no pin (see tests/test_oracle_pins.py): none -- every exported
computation is checked against closed forms, brute force, library routines,
hand-worked values or the pages' stated format rules. The conventions themselves (zero point 8, nibble
order, scale layout) are readings of the pages and are not pinned against a real
checkpoint, of which there is none here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_f64.restype = ctypes.c_double
    lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_f64.restype = ctypes.c_double
    lib.oracle_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_bf16_rne_array.argtypes = [_p, _p, _i64]
    lib.oracle_num_threads.restype = _int
    lib.oracle_set_num_threads.argtypes = [_int]
    lib.oracle_q4_unpack.argtypes = [_p, _p, _i64, _i64]
    lib.oracle_w4a16.restype = _int
    lib.oracle_w4a16.argtypes = [_p, _p, _p, _i64, _i64, _i64, _int, _p, _p]
    lib.oracle_w4a16_points.restype = _int
    lib.oracle_w4a16_points.argtypes = [_p, _p, _p, _i64, _i64, _i64, _int, _p, _p, _i64, _p, _p]
    lib.oracle_mxfp8.restype = _int
    lib.oracle_mxfp8.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
    lib.oracle_mxfp8_points.restype = _int
    lib.oracle_mxfp8_points.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p, _i64, _p, _p]
    lib.oracle_w8a16.restype = _int
    lib.oracle_w8a16.argtypes = [_p, _p, _p, _i64, _i64, _i64, _int, _p, _p]
    lib.oracle_w8a16_points.restype = _int
    lib.oracle_w8a16_points.argtypes = [_p, _p, _p, _i64, _i64, _i64, _int, _p, _p, _i64, _p, _p]
    lib.oracle_q4_repack.restype = _int
    lib.oracle_q4_repack.argtypes = [_p, _p, _i64, _i64]
    lib.oracle_q4_unrepack.restype = _int
    lib.oracle_q4_unrepack.argtypes = [_p, _p, _i64, _i64]
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


# ---- scalar decoders ---------------------------------------------------------

def bf16_to_f64(b: int) -> float:
    return _load().oracle_bf16_to_f64(int(b))


def fp16_to_f64(h: int) -> float:
    return _load().oracle_fp16_to_f64(int(h))


def e4m3_to_f64(b: int) -> float:
    return _load().oracle_e4m3_to_f64(int(b))


def e8m0_to_f64(b: int) -> float:
    return _load().oracle_e8m0_to_f64(int(b))


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_to_f64(b) for b in range(256)], dtype=np.float64)


def bf16_rne(f) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (round to nearest even)."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().oracle_bf16_rne_array(_ptr(f), _ptr(out), f.size)
    return out


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---- W4A16 -------------------------------------------------------------------

def q4_unpack(qweight: np.ndarray) -> np.ndarray:
    qweight = _c(qweight, np.int32)
    K8, N = qweight.shape
    q = np.empty((K8 * 8, N), dtype=np.uint8)
    _load().oracle_q4_unpack(_ptr(qweight), _ptr(q), N, K8 * 8)
    return q


def w4a16(x: np.ndarray, qweight: np.ndarray, scales: np.ndarray, group_size: int = 128):
    """(y64, y32) for bf16 x [M,K] (uint16 bits), GPTQ words [K/8,N], fp16 scales [K/G,N]."""
    x = _c(x, np.uint16)
    qweight = _c(qweight, np.int32)
    scales = _c(scales, np.uint16)
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K or scales.shape != (K // group_size, N):
        raise ValueError("shape mismatch")
    y64 = np.empty((M, N), dtype=np.float64)
    y32 = np.empty((M, N), dtype=np.float32)
    rc = _load().oracle_w4a16(_ptr(x), _ptr(qweight), _ptr(scales), M, N, K, group_size,
                              _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_w4a16 rejected its arguments")
    return y64, y32


def w4a16_points(x, qweight, scales, group_size, rows, cols):
    x = _c(x, np.uint16)
    qweight = _c(qweight, np.int32)
    scales = _c(scales, np.uint16)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = x.shape
    N = qweight.shape[1]
    if qweight.shape[0] * 8 != K or scales.shape != (K // group_size, N) or rows.shape != cols.shape:
        raise ValueError("shape mismatch")
    y64 = np.empty(rows.shape, dtype=np.float64)
    y32 = np.empty(rows.shape, dtype=np.float32)
    rc = _load().oracle_w4a16_points(_ptr(x), _ptr(qweight), _ptr(scales), M, N, K, group_size,
                                     _ptr(rows), _ptr(cols), rows.size, _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_w4a16_points rejected its arguments")
    return y64, y32


# ---- MXFP8 -------------------------------------------------------------------

def mxfp8(x: np.ndarray, w: np.ndarray, scales: np.ndarray):
    """(y64, y32) for bf16 x [M,K], E4M3FN codes [N,K], E8M0 codes [N,K/32]."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint8)
    scales = _c(scales, np.uint8)
    M, K = x.shape
    N = w.shape[0]
    if w.shape != (N, K) or scales.shape != (N, K // 32):
        raise ValueError("shape mismatch")
    y64 = np.empty((M, N), dtype=np.float64)
    y32 = np.empty((M, N), dtype=np.float32)
    rc = _load().oracle_mxfp8(_ptr(x), _ptr(w), _ptr(scales), M, N, K, _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_mxfp8 rejected its arguments")
    return y64, y32


def mxfp8_points(x, w, scales, rows, cols):
    x = _c(x, np.uint16)
    w = _c(w, np.uint8)
    scales = _c(scales, np.uint8)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = x.shape
    N = w.shape[0]
    if w.shape != (N, K) or scales.shape != (N, K // 32) or rows.shape != cols.shape:
        raise ValueError("shape mismatch")
    y64 = np.empty(rows.shape, dtype=np.float64)
    y32 = np.empty(rows.shape, dtype=np.float32)
    rc = _load().oracle_mxfp8_points(_ptr(x), _ptr(w), _ptr(scales), M, N, K,
                                     _ptr(rows), _ptr(cols), rows.size, _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_mxfp8_points rejected its arguments")
    return y64, y32


# ---- W8A16 (quantized vocabulary head) ---------------------------------------

def w8a16(x: np.ndarray, w: np.ndarray, scales: np.ndarray, group_size: int = 128):
    """(y64, y32) for bf16 x [M,K], int8 codes [N,K], fp16 scales [K/G,N]."""
    x = _c(x, np.uint16)
    w = _c(w, np.int8)
    scales = _c(scales, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    if w.shape != (N, K) or scales.shape != (K // group_size, N):
        raise ValueError("shape mismatch")
    y64 = np.empty((M, N), dtype=np.float64)
    y32 = np.empty((M, N), dtype=np.float32)
    rc = _load().oracle_w8a16(_ptr(x), _ptr(w), _ptr(scales), M, N, K, group_size,
                              _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_w8a16 rejected its arguments")
    return y64, y32


def w8a16_points(x, w, scales, group_size, rows, cols):
    x = _c(x, np.uint16)
    w = _c(w, np.int8)
    scales = _c(scales, np.uint16)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = x.shape
    N = w.shape[0]
    if w.shape != (N, K) or scales.shape != (K // group_size, N) or rows.shape != cols.shape:
        raise ValueError("shape mismatch")
    y64 = np.empty(rows.shape, dtype=np.float64)
    y32 = np.empty(rows.shape, dtype=np.float32)
    rc = _load().oracle_w8a16_points(_ptr(x), _ptr(w), _ptr(scales), M, N, K, group_size,
                                     _ptr(rows), _ptr(cols), rows.size, _ptr(y64), _ptr(y32))
    if rc:
        raise ValueError("oracle_w8a16_points rejected its arguments")
    return y64, y32


def rtn_quantize(w_bits: np.ndarray, bits: int, group_size: int):
    """Load-time symmetric group-wise round-to-nearest of a dense bf16 weight [N, K].

    Eole recipe "Qwen3.8-27B and native MTP speculative decoding", section
    "Optional vocabulary-head quantization" (int8 or int4, groups of 32/64/128
    along K, symmetric, round to nearest). Per group (n, g), in fp32:
        amax = max |w|,  s = fp16(amax / qmax)  with qmax = 2^(bits-1) - 1,
        q = clamp(rint(w / s), -qmax - 1, qmax)      (rint: nearest, ties to even)
    where s is used as stored (fp16 -> fp32) and a group with s == 0 gets q = 0.
    Returns (codes, scales): int8 codes [N, K] for bits = 8, GPTQ words
    [K/8, N] holding q + 8 for bits = 4; fp16 scale bits [K/G, N].
    """
    w_bits = _c(w_bits, np.uint16)
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    N, K = w_bits.shape
    G = group_size
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    W = (w_bits.astype(np.uint32) << 16).view(np.float32)       # bf16 -> fp32, exact
    Wg = W.reshape(N, K // G, G)
    qmax = np.float32(2 ** (bits - 1) - 1)
    amax = np.abs(Wg).max(axis=2)                                 # exact
    s16 = (amax / qmax).astype(np.float32).astype(np.float16)    # fp32 division, then RNE
    s = s16.astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    qf = (Wg / safe[:, :, None]).astype(np.float32)               # fp32 division
    q = np.clip(np.rint(qf), -qmax - 1, qmax)
    q = np.where((s > 0)[:, :, None], q, 0).astype(np.int32).reshape(N, K)
    scales = np.ascontiguousarray(s16.T).view(np.uint16)
    if bits == 8:
        return q.astype(np.int8), scales
    u = (q + 8).T.astype(np.uint32).reshape(K // 8, 8, N)           # [K, N] codes 0..15
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        words |= u[:, i, :] << np.uint32(4 * i)
    return words.view(np.int32), scales


# ---- device layout of packed INT4 weights ------------------------------------

def q4_repack(qweight: np.ndarray) -> np.ndarray:
    """GPTQ words [K/8, N] -> tiled words (flat int32, K*N/8 entries)."""
    qweight = _c(qweight, np.int32)
    K8, N = qweight.shape
    out = np.empty(K8 * N, dtype=np.int32)
    if _load().oracle_q4_repack(_ptr(qweight), _ptr(out), N, K8 * 8):
        raise ValueError("repack needs N % 16 == 0 and K % 128 == 0")
    return out


def q4_unrepack(tiled: np.ndarray, N: int, K: int) -> np.ndarray:
    tiled = _c(tiled, np.int32).reshape(-1)
    if tiled.size != K * N // 8:
        raise ValueError("size mismatch")
    out = np.empty((K // 8, N), dtype=np.int32)
    if _load().oracle_q4_unrepack(_ptr(tiled), _ptr(out), N, K):
        raise ValueError("unrepack needs N % 16 == 0 and K % 128 == 0")
    return out


# ---- MXFP8 tile layout ---------------------------------------------------------

def _mxfp8_tile_index(N: int, K: int):
    """For every byte offset o of the tiled buffer, the (column, K-element) of
    the [N][K] code matrix it holds."""
    if N % 16 or K % 128 or N <= 0 or K <= 0:
        raise ValueError("the MXFP8 tile layout needs N % 16 == 0 and K % 128 == 0")
    KT = K // 128
    o = np.arange(N * K, dtype=np.int64)
    tile, rem = o // 2048, o % 2048
    half, lane, byte = rem // 1024, (rem % 1024) // 16, rem % 16
    nb, kt = tile // KT, tile % KT
    col = 16 * nb + lane % 16
    k = 128 * kt + 32 * (lane // 16) + 16 * half + byte
    return col, k


def mxfp8_tile(w: np.ndarray) -> np.ndarray:
    """E4M3 codes [N, K] -> the device tile layout (flat uint8, N*K bytes).

    A layout of this library (the pages only say that weights are repacked
    once at setup: Eole recipe, section "Pack inference projections"): tiles of
    16 columns x 128 K-elements (2 KiB), column-block-major with the K-tiles of
    a column block consecutive; byte 1024*h + 16*l + b of a tile holds column
    16*nb + l%16, K-element 128*kt + 32*(l/16) + 16*h + b."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    N, K = w.shape
    col, k = _mxfp8_tile_index(N, K)
    return w[col, k]


def mxfp8_untile(tiled: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of mxfp8_tile: the flat tiled buffer back to codes [N, K]."""
    tiled = np.ascontiguousarray(tiled, dtype=np.uint8).reshape(-1)
    if tiled.size != N * K:
        raise ValueError("size mismatch")
    col, k = _mxfp8_tile_index(N, K)
    out = np.empty((N, K), dtype=np.uint8)
    out[col, k] = tiled
    return out


# ---- MXFP8 quantizer: plain and optimized round-to-nearest ---------------------

def e4m3_nearest(a) -> np.ndarray:
    """Non-negative fp32 magnitudes -> E4M3FN magnitude codes 0..0x7E: the
    nearest finite E4M3 value, ties to the even code, everything at or above
    448 saturating to 448 (the largest finite value)."""
    vals = e4m3_table()[:0x7F]                       # codes 0..0x7E, ascending values
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dl, dh = a - vals[lo], vals[hi] - a
    pick_hi = (dh < dl) | ((dh == dl) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= vals[0x7E], 0x7E, code)
    return code.astype(np.uint8)


def mxfp8_quantize(w_bits: np.ndarray, optimized: bool = True, return_choice: bool = False):
    """MXFP8 quantization of a dense bf16 weight [N, K], blocks of 32 along K.

    MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp": plain RTN to E4M3 with one
    E8M0 scale per 32 elements (opening summary), and the optimized RTN of the
    section on the quantizer's behaviours: per block the baseline E8M0 scale
    and the candidates twice and half as large are evaluated and the best one
    is kept. Baseline (OCP MX conversion rule): amax = max |v|, X0 =
    floor(log2 amax) - 8, b0 = clamp(X0 + 127, 0, 254); an all-zero block gets
    b0 = 127. Candidates, in this order: b0, b0 + 1, b0 - 1 (those within
    0..254). For a candidate b with X = b - 127, each code is E4M3_RNE(v / 2^X)
    with the sign of v, saturating at 448, and its error is the squared
    difference between v and the decoded value c * 2^X, summed over the 32
    elements in ascending order in fp32. A later candidate replaces the kept
    one only with a strictly smaller error. optimized=False keeps b0.
    Returns (codes uint8 [N, K], scales uint8 [N, K/32]) and, with
    return_choice, the index of the kept candidate per block (0, 1, 2).
    """
    w_bits = _c(w_bits, np.uint16)
    N, K = w_bits.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    W = ((w_bits.astype(np.uint32) << 16).view(np.float32)).reshape(N, K // 32, 32)
    A = np.abs(W)
    amax = A.max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, np.float32(1)).astype(np.float64))
    b0 = np.where(amax > 0, np.clip((ex - 1) - 8 + 127, 0, 254), 127).astype(np.int64)
    table = e4m3_table()
    sign = np.signbit(W)

    def candidate(b):
        X = (b - 127)[:, :, None]
        scaled = np.ldexp(A, -X).astype(np.float32)               # exact power-of-two step
        mag = e4m3_nearest(scaled)
        d = np.ldexp(table[mag], X).astype(np.float32)            # decoded magnitude, exact
        d = np.where(sign, -d, d).astype(np.float32)
        diff = (W - d).astype(np.float32)
        sq = (diff * diff).astype(np.float32)
        err = np.zeros((N, K // 32), dtype=np.float32)
        for i in range(32):
            err = (err + sq[:, :, i]).astype(np.float32)
        codes = (mag | (sign.astype(np.uint8) << np.uint8(7))).astype(np.uint8)
        return codes, err

    # near the top of the bf16 range a decoded value or a squared difference can
    # overflow fp32 to infinity; that is the defined fp32 result of these steps
    with np.errstate(over="ignore", under="ignore"):
        return _mxfp8_select(candidate, b0, optimized, N, K, return_choice)


def _mxfp8_select(candidate, b0, optimized, N, K, return_choice):
    best_codes, best_err = candidate(b0)
    best_b = b0.copy()
    choice = np.zeros_like(b0)
    if optimized:
        for k, step in ((1, 1), (2, -1)):
            b = b0 + step
            ok = (b >= 0) & (b <= 254)
            codes, err = candidate(np.clip(b, 0, 254))
            take = ok & (err < best_err)
            best_codes = np.where(take[:, :, None], codes, best_codes)
            best_err = np.where(take, err, best_err)
            best_b = np.where(take, b, best_b)
            choice = np.where(take, k, choice)
    out = (best_codes.reshape(N, K), best_b.astype(np.uint8))
    return out + (choice,) if return_choice else out


# ---- setup-time projection fusion and compressed-tensors ingest ----------------

def fuse_incompatibility(parts, bits: int, group_size: int):
    """Why a list of quantized projections cannot be fused, or None if it can.

    Eole recipe "Qwen3.8-27B and native MTP speculative decoding", section
    "Pack inference projections": projections that read the same input are
    packed together at setup, before the kernel repack, without requantizing;
    pairs that do not fit keep their own projections. Read here as: same
    weight format (bits), same K, same group size, and every width a multiple
    of the 16-column tile of the packed layout. ``parts`` holds
    (weights, scales) pairs in the formats of ``fuse_projections``.
    """
    if bits not in (4, 8):
        return "bits must be 4 or 8"
    if not parts:
        return "no projections"
    Ks, Ns = [], []
    for w, s in parts:
        w, s = np.asarray(w), np.asarray(s)
        if bits == 4:
            K, N = w.shape[0] * 8, w.shape[1]
        else:
            N, K = w.shape
        if s.shape[1] != N or K % group_size or s.shape[0] != K // group_size:
            return "scales do not match the weights or the group size"
        Ks.append(K)
        Ns.append(N)
    if len(set(Ks)) != 1:
        return "projections read inputs of different K"
    if any(n % 16 for n in Ns):
        return "a width is not a multiple of 16"
    return None


def fuse_projections(parts, bits: int, group_size: int):
    """Concatenate quantized projections along N, in the order given.

    Eole recipe, section "Pack inference projections" (K/V/Q and gate/up
    packed before the repack, no requantization). Output column n of the
    fused layer is column n - off_p of part p, where off_p is the sum of the
    widths before it, so y_fused = [y_0 | y_1 | ...] exactly.
      bits 4: GPTQ words [K/8, N_p] -> [K/8, sum N_p]   (columns appended)
      bits 8: int8 codes [N_p, K]   -> [sum N_p, K]     (rows appended)
      scales fp16 [K/G, N_p]       -> [K/G, sum N_p]   (columns appended)
    """
    why = fuse_incompatibility(parts, bits, group_size)
    if why:
        raise ValueError(why)
    ws = [np.asarray(w) for w, _ in parts]
    ss = [_c(s, np.uint16) for _, s in parts]
    wf = np.concatenate([_c(w, np.int32) for w in ws], axis=1) if bits == 4 else \
        np.concatenate([_c(w, np.int8) for w in ws], axis=0)
    return wf, np.concatenate(ss, axis=1)


def ct_to_gptq(weight_packed: np.ndarray, weight_scale: np.ndarray):
    """Compressed-tensors W4A16 [N, K/8] words and [N, K/G] scales -> GPTQ layout.

    Eole recipe, section "Compressed-tensors INT4 layout": the converter
    transposes the packed INT4 words and the scales into the GPTQ layout and
    does not dequantize. The words themselves are unchanged, so nibble i of
    compressed-tensors word [n][j] is the code of row 8j + i, column n, as in
    GPTQ word [j][n]. Returns (qweight int32 [K/8, N], scales fp16 bits
    [K/G, N]).
    """
    wp = _c(weight_packed, np.int32)
    sc = _c(weight_scale, np.uint16)
    if wp.ndim != 2 or sc.ndim != 2 or sc.shape[0] != wp.shape[0]:
        raise ValueError("weight_packed [N, K/8] and weight_scale [N, K/G] expected")
    return np.ascontiguousarray(wp.T), np.ascontiguousarray(sc.T)


# ---- the parity gate ---------------------------------------------------------

def gate(out_bits: np.ndarray, y_ref: np.ndarray, rel_tol: float = 2e-2):
    """max |fp32(out) - y_ref| <= rel_tol * RMS(y_ref) over all outputs.

    Returns (ok, max_err, rms). The tolerance is the one the layer's accuracy
    target states for bf16 outputs against an fp32-accumulated reference.
    """
    out = bf16_bits_to_f64(out_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    err = float(np.max(np.abs(out - y_ref))) if y_ref.size else 0.0
    return err <= rel_tol * rms, err, rms
