"""Seeded synthetic inputs for the weight-only quantized linear layer.

This module is the only code shared by the CPU oracle's tests and the GPU path's
tests and benchmark. It produces input *bytes* only: activations in bf16, GPTQ
packed INT4 words with fp16 group scales, and MXFP8 (E4M3 element codes with an
E8M0 scale per 32 K-elements). It contains none of the layer's arithmetic: no
unpacking, no dequantisation, no dot products, no output rounding.

Formats produced (each the plainest reading of the cited page where it leaves a detail open):

* W4A16, GPTQ layout -- GPTQ INT4 card "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16",
  section "Quantization contract": symmetric INT4, group size 128, desc_act off,
  packed int32. ``qweight[j, n]`` holds q[8j+i, n] in bits 4i..4i+3 (i = 0 is the
  least significant nibble); ``scales[g, n]`` is fp16 for K-group g = k // G.
  Eole recipe "Qwen3.8-27B and native MTP speculative decoding", section
  "Compressed-tensors INT4 layout", accepts group sizes 32, 64 and 128.
* MXFP8 -- MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp", opening summary and
  section "8. License and attribution": OCP Microscaling, 8-bit elements with an
  E8M0 shared scale per 32-element block, produced by plain round-to-nearest
  without calibration. Elements are E4M3FN, blocks run along K within a row n,
  weights are stored [N, K] and scales [N, K/32].

* W8A16, the quantized vocabulary head -- Eole recipe "Qwen3.8-27B and native
  MTP speculative decoding", section "Optional vocabulary-head quantization"
  (int8, symmetric group-wise round to nearest, groups along K): int8 codes
  stored [N, K], fp16 scales [K/G, N]. Dense bf16 weights [N, K] feed the
  load-time quantizer.

Value distributions: x ~ N(0, 1) rounded to bf16; q uniform on [0, 15]; scales
uniform on [0.002, 0.02] rounded to fp16; MXFP8 weights come from an N(0, 1)
matrix. Draw order from one ``numpy.random.default_rng(seed)``: x, then q (or the
fp32 matrix W), then scales.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits", "fp16_bits", "pack_gptq", "e4m3_encode_rne", "mxfp8_quantize_rtn",
    "gen_w4a16", "gen_mxfp8", "gen_w8a16", "gen_dense_bf16", "W4A16Inputs", "MXFP8Inputs",
    "W8A16Inputs", "WORKLOADS", "sha256", "FusionInputs", "gen_fusion", "gen_ct_w4a16", "FUSIONS",
]


def bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite values only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def fp16_bits(a) -> np.ndarray:
    """fp32/fp64 -> IEEE binary16 bit patterns (numpy's round to nearest even)."""
    return np.ascontiguousarray(a).astype(np.float16).view(np.uint16)


def pack_gptq(q: np.ndarray) -> np.ndarray:
    """Pack uint4 codes q[K, N] into GPTQ words [K/8, N] (nibble i = row 8j+i)."""
    q = np.asarray(q, dtype=np.uint32)
    K, N = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    if q.max(initial=0) > 15:
        raise ValueError("codes must lie in [0, 15]")
    q = q.reshape(K // 8, 8, N)
    w = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        w |= q[:, i, :] << np.uint32(4 * i)
    return w.view(np.int32)


def e4m3_encode_rne(v) -> np.ndarray:
    """fp32 values -> OCP E4M3FN codes, round to nearest even, saturating at +-448.

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds
    the subnormals m/8 * 2^-6; 0x7F/0xFF are NaN; there is no infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(v), 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2^-9; rounding up to 8 * 2^-9 yields the
    # smallest normal (code 0x08) by construction
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        frac, ex = np.frexp(a[nrm])          # a = frac * 2^ex, frac in [0.5, 1)
        e = ex - 1                           # floor(log2 a)
        m = np.rint((a[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        e = e + carry
        m = np.where(carry, 0, m)
        code[nrm] = ((e + 7) << 3) | m
    code = np.minimum(code, 0x7E)            # 448 is the largest finite value
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def mxfp8_quantize_rtn(W: np.ndarray, block: int = 32):
    """Plain RTN MXFP8 of W[N, K] with blocks of ``block`` along K.

    Per block: amax = max|v|; an all-zero block gets scale code 127 and zero
    elements; otherwise the shared exponent is X = floor(log2 amax) - 8 (8 is the
    largest E4M3 normal exponent), the E8M0 code is clamp(X + 127, 0, 254) and
    each element is E4M3_RNE(v / 2^X), saturating at 448.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    Wb = W.reshape(N, K // block, block).astype(np.float64)
    amax = np.abs(Wb).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = (ex - 1) - 8
    sc = np.clip(X + 127, 0, 254)
    sc = np.where(amax > 0, sc, 127).astype(np.uint8)
    scaled = Wb / np.ldexp(1.0, sc.astype(np.int64) - 127)[:, :, None]
    codes = e4m3_encode_rne(scaled).reshape(N, K)
    return codes, sc


def sha256(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@dataclass
class W4A16Inputs:
    M: int
    K: int
    N: int
    G: int
    x: np.ndarray        # uint16 bf16 bits [M, K]
    qweight: np.ndarray  # int32 GPTQ words [K/8, N]
    scales: np.ndarray   # uint16 fp16 bits [K/G, N]
    q: np.ndarray = field(repr=False, default=None)  # uint8 codes [K, N] (kept for pins)

    def digest(self) -> str:
        return sha256(self.x, self.qweight, self.scales)


@dataclass
class W8A16Inputs:
    M: int
    K: int
    N: int
    G: int
    x: np.ndarray       # uint16 bf16 bits [M, K]
    w: np.ndarray       # int8 codes [N, K]
    scales: np.ndarray  # uint16 fp16 bits [K/G, N]

    def digest(self) -> str:
        return sha256(self.x, self.w, self.scales)


@dataclass
class MXFP8Inputs:
    M: int
    K: int
    N: int
    x: np.ndarray       # uint16 bf16 bits [M, K]
    w: np.ndarray       # uint8 E4M3FN codes [N, K]
    scales: np.ndarray  # uint8 E8M0 codes [N, K/32]

    def digest(self) -> str:
        return sha256(self.x, self.w, self.scales)


def _x(rng, M, K, kind):
    if kind == "intexact":
        return bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    return bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def gen_w4a16(seed: int, M: int, K: int, N: int, G: int = 128, kind: str = "random",
              keep_q: bool = False) -> W4A16Inputs:
    """Seeded W4A16 inputs.

    kind="random":   x ~ N(0,1) in bf16, q ~ U{0..15}, s ~ U[0.002, 0.02] in fp16.
    kind="intexact": x ~ U{-4..4}, q ~ U{0..15}, s = 1.0, so every partial sum is
                     an integer below 2^24 and the exact result is unique.
    """
    if K % G or K % 8:
        raise ValueError("K must be a multiple of G and of 8")
    rng = np.random.default_rng(seed)
    x = _x(rng, M, K, kind)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    if kind == "intexact":
        s = fp16_bits(np.ones((K // G, N), dtype=np.float32))
    else:
        s = fp16_bits(rng.uniform(0.002, 0.02, size=(K // G, N)).astype(np.float32))
    return W4A16Inputs(M, K, N, G, x, pack_gptq(q), s, q if keep_q else None)


def gen_mxfp8(seed: int, M: int, K: int, N: int, kind: str = "random") -> MXFP8Inputs:
    """Seeded MXFP8 inputs.

    kind="random":   x ~ N(0,1) in bf16; W ~ N(0,1) quantised by plain RTN.
    kind="intexact": x ~ U{-4..4}; element codes of the integers -8..8 with scale
                     code 127 (2^0), so the exact result is an integer.
    """
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    x = _x(rng, M, K, kind)
    if kind == "intexact":
        ints = rng.integers(-8, 9, size=(N, K)).astype(np.float64)
        w = e4m3_encode_rne(ints)
        sc = np.full((N, K // 32), 127, dtype=np.uint8)
    else:
        W = rng.standard_normal((N, K), dtype=np.float32)
        w, sc = mxfp8_quantize_rtn(W)
    return MXFP8Inputs(M, K, N, x, w, sc)


def gen_w8a16(seed: int, M: int, K: int, N: int, G: int = 128, kind: str = "random") -> W8A16Inputs:
    """Seeded W8A16 inputs.

    kind="random":   x ~ N(0,1) in bf16, q ~ U{-128..127}, s ~ U[2e-4, 2e-3] in fp16
                     (the scale range of int8 round-to-nearest of N(0, 0.02) weights).
    kind="intexact": x ~ U{-4..4}, s = 1.0: integer partial sums below 2^24.
    """
    if K % G:
        raise ValueError("K must be a multiple of G")
    rng = np.random.default_rng(seed)
    x = _x(rng, M, K, kind)
    w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    if kind == "intexact":
        s = fp16_bits(np.ones((K // G, N), dtype=np.float32))
    else:
        s = fp16_bits(rng.uniform(2e-4, 2e-3, size=(K // G, N)).astype(np.float32))
    return W8A16Inputs(M, K, N, G, x, w, s)


def gen_dense_bf16(seed: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """Seeded dense weights [N, K] ~ N(0, std^2) as bf16 bits (input of the quantizer)."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(std))


@dataclass
class FusionInputs:
    M: int
    K: int
    G: int
    bits: int
    widths: list
    x: np.ndarray        # uint16 bf16 bits [M, K]
    parts: list          # [(weights, scales)]: GPTQ words [K/8, N_p] or int8 [N_p, K]; fp16 bits [K/G, N_p]


def gen_fusion(seed: int, M: int, K: int, widths, G: int = 128, bits: int = 4,
               kind: str = "random") -> FusionInputs:
    """Seeded projections that share one x, each drawn like gen_w4a16 / gen_w8a16."""
    rng = np.random.default_rng(seed)
    x = _x(rng, M, K, kind)
    parts = []
    for n in widths:
        if bits == 4:
            w = pack_gptq(rng.integers(0, 16, size=(K, n), dtype=np.uint8))
            lo, hi = 0.002, 0.02
        else:
            w = rng.integers(-128, 128, size=(n, K), dtype=np.int8)
            lo, hi = 2e-4, 2e-3
        if kind == "intexact":
            sc = fp16_bits(np.ones((K // G, n), dtype=np.float32))
        else:
            sc = fp16_bits(rng.uniform(lo, hi, size=(K // G, n)).astype(np.float32))
        parts.append((w, sc))
    return FusionInputs(M, K, G, bits, list(widths), x, parts)


def gen_ct_w4a16(seed: int, N: int, K: int, G: int = 128):
    """Seeded compressed-tensors W4A16 tensors: uniformly random int32 words
    [N, K/8] (every nibble U{0..15}) and fp16 scales [N, K/G] ~ U[0.002, 0.02]."""
    rng = np.random.default_rng(seed)
    words = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    sc = fp16_bits(rng.uniform(0.002, 0.02, size=(N, K // G)).astype(np.float32))
    return words, sc


# Projections fused at setup: K/V/Q of attention (K and V 4 x 256 wide, Q 24 x 256,
# the head counts of the GPTQ card's "Model facts" with head_dim 256) and the MLP's
# gate and up (two 17408-wide halves), at decode (M=1) and verify (M=5) sizes.
FUSIONS = {
    "kvq_m1":     dict(M=1, K=5120, widths=[1024, 1024, 6144], seed=701),
    "kvq_m5":     dict(M=5, K=5120, widths=[1024, 1024, 6144], seed=702),
    "gate_up_m1": dict(M=1, K=5120, widths=[17408, 17408], seed=703),
    "gate_up_m5": dict(M=5, K=5120, widths=[17408, 17408], seed=704),
}


# Named workloads: single-stream decode (M=1), MTP verify chunks (M = 1 + drafts),
# and batched verify (32 streams x (1 + 3) tokens). K = 5120 is the hidden size in
# the GPTQ card's "Model facts"; 17408 is a synthetic MLP width.
WORKLOADS = {
    "tiny":          dict(op="w4a16", M=1,   K=512,   N=256,   seed=101),
    "decode_n5120":  dict(op="w4a16", M=1,   K=5120,  N=5120,  seed=201),
    "decode_n6144":  dict(op="w4a16", M=1,   K=5120,  N=6144,  seed=202),
    "decode_n1024":  dict(op="w4a16", M=1,   K=5120,  N=1024,  seed=203),
    "verify5_up":    dict(op="w4a16", M=5,   K=5120,  N=17408, seed=301),
    "verify5_down":  dict(op="w4a16", M=5,   K=17408, N=5120,  seed=302),
    "verify3_up":    dict(op="w4a16", M=3,   K=5120,  N=17408, seed=303),
    "verify3_down":  dict(op="w4a16", M=3,   K=17408, N=5120,  seed=304),
    "batch128_up":   dict(op="w4a16", M=128, K=5120,  N=17408, seed=401),
    "batch128_down": dict(op="w4a16", M=128, K=17408, N=5120,  seed=402),
    "mxfp8_m1":      dict(op="mxfp8", M=1,   K=5120,  N=5120,  seed=501),
    "mxfp8_m5":      dict(op="mxfp8", M=5,   K=5120,  N=5120,  seed=502),
    "mxfp8_m128":    dict(op="mxfp8", M=128, K=5120,  N=5120,  seed=503),
    # quantized vocabulary head: N = 248320 (about 248k entries, a multiple of 256)
    "vocab_w8_m1":   dict(op="w8a16", M=1,   K=5120,  N=248320, seed=601),
    "vocab_w4_m1":   dict(op="w4a16", M=1,   K=5120,  N=248320, seed=602),
    # the smaller group sizes the compressed-tensors layout allows (32 and 64)
    "decode_n6144_g32":  dict(op="w4a16", M=1,   K=5120, N=6144,  seed=211, G=32),
    "decode_n6144_g64":  dict(op="w4a16", M=1,   K=5120, N=6144,  seed=212, G=64),
    "verify5_up_g32":    dict(op="w4a16", M=5,   K=5120, N=17408, seed=311, G=32),
    "verify5_up_g64":    dict(op="w4a16", M=5,   K=5120, N=17408, seed=312, G=64),
    "batch128_up_g32":   dict(op="w4a16", M=128, K=5120, N=17408, seed=411, G=32),
    "batch128_up_g64":   dict(op="w4a16", M=128, K=5120, N=17408, seed=412, G=64),
}


def gen_workload(name: str, kind: str = "random"):
    w = WORKLOADS[name]
    G = w.get("G", 128)
    if w["op"] == "w4a16":
        return gen_w4a16(w["seed"], w["M"], w["K"], w["N"], G, kind)
    if w["op"] == "w8a16":
        return gen_w8a16(w["seed"], w["M"], w["K"], w["N"], G, kind)
    return gen_mxfp8(w["seed"], w["M"], w["K"], w["N"], kind)
