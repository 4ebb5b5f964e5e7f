"""GPU parity: every HIP kernel through the C ABI against the CPU oracle on the
same seeded inputs.

Tolerance (random inputs): max |fp32(out) - y_ref| <= 2e-2 * RMS(y_ref) against
both the fp64-summed oracle and the fp32-sequential oracle. Integer-valued inputs
have one exact answer: outputs must equal bf16_RNE(exact) bit for bit. Repack is
bit-exact. Small shapes are compared element by element; the full-size
workloads (in the launch configuration the benchmark times) over every output,
including the vocabulary heads (N = 248320).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    import spec_verify_amd as svq
    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    svq.lib()
    yield


def _say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_w4a16(inp, kernel=0, out=None):
    import spec_verify_amd as svq
    qw = dev(inp.qweight)
    tiled = svq.q4_repack(qw)
    o = svq.w4a16_gemm(dev(inp.x), tiled, dev(inp.scales), inp.N, inp.G, out=out, kernel=kernel)
    torch.cuda.synchronize()
    return host_bits(o), tiled


def run_mxfp8(inp, kernel=0):
    import spec_verify_amd as svq
    o = svq.mxfp8_gemm(dev(inp.x), svq.mxfp8_repack(dev(inp.w)), dev(inp.scales), kernel=kernel)
    torch.cuda.synchronize()
    return host_bits(o)


def assert_gate(out, y64, y32, label):
    ok64, e64, rms = oracle.gate(out, y64)
    ok32, e32, _ = oracle.gate(out, y32.astype(np.float64))
    assert ok64 and ok32, f"{label}: err64={e64:.4g} err32={e32:.4g} rms={rms:.4g} ratio={e64 / max(rms, 1e-30):.4g}"


# ---- repack -------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 512), (5120, 5120), (1024, 17408)])
def test_repack_bit_exact(N, K):
    _say("repack", N, K)
    inp = synth.gen_w4a16(7 + N, 1, K, N)
    import spec_verify_amd as svq
    got = svq.q4_repack(dev(inp.qweight)).cpu().numpy()
    ref = oracle.q4_repack(inp.qweight)
    np.testing.assert_array_equal(got, ref)
    if N * K <= 1 << 20:
        np.testing.assert_array_equal(oracle.q4_unrepack(got, N, K), inp.qweight)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (256, 640), (5120, 5120), (1024, 17408)])
def test_mxfp8_repack_bit_exact(N, K):
    _say("mxfp8 repack", N, K)
    rng = np.random.default_rng(17 + N + K)
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    import spec_verify_amd as svq
    got = svq.mxfp8_repack(torch.from_numpy(w).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.mxfp8_tile(w))


# ---- W4A16 small shapes, every kernel -------------------------------------------

KNAME = {1: "dot2", 2: "skinny", 3: "wide"}


def _ids(cases):
    return ["-".join([KNAME[c[0]]] + [str(v) for v in c[1:]]) for c in cases]


W4_CASES = (
    [(1, m, K, N, G) for m in (1, 2, 3, 5, 8) for (K, N) in ((512, 48), (1280, 32)) for G in (32, 64, 128)]
    + [(2, m, K, N, G) for m in (1, 3, 5, 11, 16) for (K, N) in ((512, 48), (1280, 32)) for G in (32, 64, 128)]
    # the skinny kernel's packed rows at G = 32 / 64: every row count at the slot
    # boundaries (4 rows per slot up to M = 4, 8 rows up to M = 8, unpacked from 9),
    # and K = 17408 split three ways over workgroups
    + [(2, m, K, N, G) for m in (2, 4, 6, 7, 8, 9) for (K, N) in ((512, 48), (1280, 32)) for G in (32, 64)]
    + [(2, m, 17408, 64, G) for m in (1, 4, 5, 8) for G in (32, 64)]
    + [(3, m, K, N, G) for m in (1, 17, 64, 65, 128, 130) for (K, N) in ((1024, 272), (2560, 128)) for G in (32, 128)]
    + [(3, 33, 640, 16, 64)]
    # dot2 with more column blocks than compute units (456, 336 and 576 blocks)
    + [(1, m, K, N, G) for (m, K, N, G) in ((1, 1280, 7296, 128), (3, 1280, 7296, 32), (2, 1280, 5376, 128),
                                            (8, 640, 5376, 64), (5, 1280, 9216, 128), (1, 1280, 9216, 32))]
)

# dot2 shapes that run the narrow-unit GEMV on a 256-CU part (M <= 2, fewer 16-column
# blocks than CUs, at least one 4-column unit per CU): ragged groups of four tiles
# (K = 1280, 640), one to four units per workgroup, every group size, long K
W4_NARROW = [(1, m, K, N, G) for (m, K, N, G) in (
    (1, 1280, 1024, 128), (2, 1280, 1040, 32), (1, 5120, 4080, 64), (2, 640, 2064, 32),
    (1, 17408, 1024, 128), (1, 5120, 1024, 32), (2, 5120, 3088, 64))]


@pytest.mark.parametrize("kernel,M,K,N,G", W4_CASES, ids=_ids(W4_CASES))
def test_w4a16_random(kernel, M, K, N, G):
    _say("w4a16 random kernel", kernel, "M K N G", M, K, N, G)
    inp = synth.gen_w4a16(1000 + 7 * M + K + N + G, M, K, N, G)
    out, _ = run_w4a16(inp, kernel)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    assert_gate(out, y64, y32, f"kernel {kernel} M{M} K{K} N{N} G{G}")


@pytest.mark.parametrize("kernel,M,K,N,G", W4_NARROW, ids=_ids(W4_NARROW))
def test_w4a16_narrow(kernel, M, K, N, G):
    import spec_verify_amd as svq
    _say("w4a16 narrow M K N G", M, K, N, G)
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("shapes chosen for a 256-CU part")
    assert svq.w4a16_kernel_name(M, N, K, G, kernel=1) == "w4a16_narrow_kernel"
    inp = synth.gen_w4a16(2000 + 7 * M + K + N + G, M, K, N, G)
    out, _ = run_w4a16(inp, kernel)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    assert_gate(out, y64, y32, f"narrow M{M} K{K} N{N} G{G}")


# fp16 scales at the ends of their range, per (group, column): zero, the smallest
# subnormal (2^-24), the smallest normal (2^-14), the largest finite value, negative
# values and one; the kernels convert the scale to fp32 exactly, so the gate against
# the fp64 and fp32 oracles holds as for ordinary scales
EXTREME_SCALES = np.array([0x0000, 0x0001, 0x0400, 0x7BFF, 0xB800, 0x3C00, 0x8001, 0x03FF], dtype=np.uint16)


@pytest.mark.parametrize("kernel,M,N", [(1, 1, 64), (1, 1, 1024), (1, 3, 64), (2, 3, 64), (2, 5, 64), (3, 40, 64)],
                         ids=["dot2-1", "narrow-1", "dot2-3", "skinny-3", "skinny-5", "wide-40"])
@pytest.mark.parametrize("G", [32, 128])
def test_w4a16_extreme_scales(kernel, M, N, G):
    _say("w4a16 extreme scales kernel", kernel, "M", M, "N", N, "G", G)
    K = 512
    inp = synth.gen_w4a16(4000 + 13 * M + G, M, K, N, G)
    rng = np.random.default_rng(4100 + M + G)
    inp.scales = EXTREME_SCALES[rng.integers(0, len(EXTREME_SCALES), size=inp.scales.shape)]
    out, _ = run_w4a16(inp, kernel)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    assert_gate(out, y64, y32, f"extreme scales kernel {kernel} M{M} G{G}")


W4_EXACT = [
    (1, 1, 1024, 32, 128), (1, 5, 1024, 32, 32), (1, 8, 640, 48, 64),
    (2, 1, 1024, 32, 128), (2, 7, 1024, 32, 32), (2, 16, 640, 48, 64),
    # the skinny kernel's packed rows: 4-row slots (G = 32), 8-row slots (G = 64), two chains (G = 32)
    (2, 3, 1024, 32, 32), (2, 5, 1024, 48, 64), (2, 8, 640, 32, 32),
    (3, 128, 1024, 272, 128), (3, 40, 1024, 144, 32), (3, 130, 640, 128, 64),
]


@pytest.mark.parametrize("kernel,M,K,N,G", W4_EXACT, ids=_ids(W4_EXACT))
def test_w4a16_integer_exact(kernel, M, K, N, G):
    _say("w4a16 intexact kernel", kernel, "M K N G", M, K, N, G)
    inp = synth.gen_w4a16(77 + M, M, K, N, G, kind="intexact", keep_q=True)
    out, _ = run_w4a16(inp, kernel)
    xi = oracle.bf16_bits_to_f64(inp.x).astype(np.int64)
    exact = xi @ (inp.q.astype(np.int64) - 8)
    np.testing.assert_array_equal(out, oracle.bf16_rne(exact.astype(np.float32)))


# ---- W4A16 full-size workloads ---------------------------------------------------

def _sample(M, N, n, seed):
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M, n)
    cols = rng.integers(0, N, n)
    rows[:4] = [0, M - 1, 0, M - 1]
    cols[:4] = [0, 0, N - 1, N - 1]
    return rows, cols


@pytest.mark.parametrize("name", ["tiny", "decode_n5120", "decode_n6144", "decode_n1024",
                                  "verify5_up", "verify5_down", "verify3_up", "verify3_down",
                                  "batch128_up", "batch128_down",
                                  # the compressed-tensors group sizes at decode, verify and batch shapes
                                  "decode_n6144_g32", "decode_n6144_g64", "verify5_up_g32",
                                  "verify5_up_g64", "batch128_up_g32", "batch128_up_g64"])
def test_w4a16_workloads(name):
    w = synth.WORKLOADS[name]
    _say("w4a16 workload", name, w)
    inp = synth.gen_workload(name)
    out, tiled = run_w4a16(inp)
    # every output against the full oracle (fp64 and fp32-sequential sums); at
    # M = 128 that is 2.2 M outputs per projection, a few seconds on the host
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, inp.G)
    assert_gate(out, y64, y32, name)
    # the repacked weights of the full-size run are the oracle's, bit for bit
    np.testing.assert_array_equal(tiled.cpu().numpy(), oracle.q4_repack(inp.qweight))


# Skinny shapes whose workgroups own several column blocks on a 256-CU part (one x
# stage of 59 KB per workgroup: two workgroups per CU): N = 5136 -> 2 blocks per
# workgroup, N = 6416 -> 4; both leave a last workgroup with a single block, and both
# split K = 17408 three ways (the split path reduces per block).
@pytest.mark.parametrize("N", [5136, 6416])
def test_w4a16_skinny_multiblock(N):
    M, K = 5, 17408
    _say("w4a16 skinny multi-block M K N", M, K, N)
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("shapes chosen for a 256-CU part")
    inp = synth.gen_w4a16(3000 + N, M, K, N, 128)
    out, _ = run_w4a16(inp, 2)
    rows, cols = _sample(M, N, 1200, N)
    cols[4:36] = np.arange(N - 32, N)        # the last workgroup's single block and its neighbour
    y64, y32 = oracle.w4a16_points(inp.x, inp.qweight, inp.scales, 128, rows, cols)
    sel = out[rows, cols]
    ok, err, rms = oracle.gate(sel, y64)
    assert ok, f"N={N}: err={err:.4g} rms={rms:.4g}"
    assert oracle.gate(sel, y32.astype(np.float64))[0]
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(out)))


# ---- MXFP8 -------------------------------------------------------------------------

MX_CASES = (
    [(1, m, K, N) for m in (1, 2, 5, 8) for (K, N) in ((512, 128), (1280, 144))]
    + [(2, m, K, N) for m in (1, 5, 16) for (K, N) in ((512, 128), (1280, 144))]
    + [(3, m, K, N) for m in (1, 17, 64, 128, 130) for (K, N) in ((1024, 272), (640, 128))]
)


@pytest.mark.parametrize("kernel,M,K,N", MX_CASES, ids=_ids(MX_CASES))
def test_mxfp8_random(kernel, M, K, N):
    _say("mxfp8 random kernel", kernel, "M K N", M, K, N)
    inp = synth.gen_mxfp8(2000 + M + K + N, M, K, N)
    out = run_mxfp8(inp, kernel)
    y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    assert_gate(out, y64, y32, f"mxfp8 kernel {kernel} M{M} K{K} N{N}")


MX_EXACT = [(1, 1), (1, 8), (2, 3), (2, 16), (3, 64), (3, 130)]


@pytest.mark.parametrize("kernel,M", MX_EXACT, ids=_ids(MX_EXACT))
def test_mxfp8_integer_exact(kernel, M):
    _say("mxfp8 intexact kernel", kernel, "M", M)
    inp = synth.gen_mxfp8(88 + M, M, 640, 272, kind="intexact")
    out = run_mxfp8(inp, kernel)
    table = oracle.e4m3_table()
    exact = oracle.bf16_bits_to_f64(inp.x).astype(np.int64) @ table[inp.w].astype(np.int64).T
    np.testing.assert_array_equal(out, oracle.bf16_rne(exact.astype(np.float32)))


@pytest.mark.parametrize("kernel", [1, 2, 3], ids=["dot2", "skinny", "wide"])
@pytest.mark.parametrize("scale_code", [127, 120, 131, 0, 1])
def test_mxfp8_hardware_decode_all_codes(kernel, scale_code):
    """Column n holds E4M3 code n at every K; x is one-hot, so y[0, n] is the
    decoded value of code n times 2^(scale-127): all 254 finite codes through
    the kernel's own conversion, against the oracle's decoder. Codes 0 and 1 are
    the smallest E8M0 scales (2^-127 is an fp32 subnormal): the products then
    reach the bf16 subnormal range, which must not be flushed."""
    _say("mxfp8 all codes kernel", kernel, "scale", scale_code)
    N, K = 256, 128
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0                       # NaN codes are not inputs
    w = np.repeat(codes[:, None], K, axis=1)
    sc = np.full((N, K // 32), scale_code, dtype=np.uint8)
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, 37] = 0x3F80                             # 1.0
    inp = synth.MXFP8Inputs(1, K, N, x, w, sc)
    out = run_mxfp8(inp, kernel)
    vals = np.array([oracle.e4m3_to_f64(int(c)) for c in codes]) * oracle.e8m0_to_f64(scale_code)
    vals = vals + 0.0    # a sum that starts from +0 turns the code 0x80 (-0) into +0
    want = oracle.bf16_rne(vals.astype(np.float32))
    # A product below half the smallest bf16 subnormal (codes 0x81..0x84 at scale
    # 2^-127) is a signed zero already in the converted bf16 weight, and
    # +0 + (-0) = +0; the exact value rounds to -0 only at the output. Where the
    # expected result is a zero, either sign is accepted; everything else (the bf16
    # subnormal outputs included) must match bit for bit.
    zero = (want & 0x7FFF) == 0
    np.testing.assert_array_equal(out[0][~zero], want[~zero])
    assert np.all((out[0][zero] & 0x7FFF) == 0)


TINY_CASES = [(1, 1, 144), (1, 4, 144), (2, 5, 144), (2, 16, 144), (3, 128, 272)]


@pytest.mark.parametrize("kernel,M,N", TINY_CASES, ids=_ids(TINY_CASES))
@pytest.mark.parametrize("codes", [(0,), (1,), (2,), (0, 1, 2, 3, 120, 127)], ids=["b0", "b1", "b2", "mixed"])
def test_mxfp8_tiny_scales_random(kernel, M, N, codes):
    """E8M0 codes b <= 2 put E4M3 * 2^(b-127) (a multiple of 2^(b-136)) below
    2^-126, where the bf16 operand the kernels build has subnormal spacing
    2^-133: such an element moves by up to 2^-134 (code 0x05 at b = 0, 5 * 2^-136,
    becomes 2^-133); at b >= 3 every element is exact. Random x, every finite
    E4M3 code, scales drawn from `codes` per block: the result passes the gate,
    and every output lies within the bound that follows from that operand
    rounding, fp32 accumulation and the bf16 output rounding."""
    _say("mxfp8 tiny scales kernel", kernel, "M N", M, N, "codes", codes)
    K = 1280
    rng = np.random.default_rng(4100 + 7 * kernel + M + len(codes) + codes[0])
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x3F                  # NaN codes are not inputs
    sc = rng.choice(np.array(codes, dtype=np.uint8), size=(N, K // 32))
    inp = synth.MXFP8Inputs(M, K, N, x, w, sc)
    out = run_mxfp8(inp, kernel)
    y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    assert_gate(out, y64, y32, f"mxfp8 tiny scales {codes} kernel {kernel} M{M}")
    xs = np.abs(oracle.bf16_bits_to_f64(x))                              # [M, K]
    table = oracle.e4m3_table()
    wv = table[w] * np.vectorize(oracle.e8m0_to_f64)(np.repeat(sc, 32, axis=1))  # [N, K] exact
    tiny = np.repeat(sc <= 2, 32, axis=1)
    e_op = 2.0 ** -134 * (xs @ tiny.T.astype(np.float64))                # operand rounding
    e_acc = K * 2.0 ** -24 / (1 - K * 2.0 ** -24) * (xs @ np.abs(wv).T) + K * 2.0 ** -150
    bound = e_op + e_acc + (np.abs(y64) + e_op + e_acc) * 2.0 ** -8 + 2.0 ** -134
    err = np.abs(oracle.bf16_bits_to_f64(out) - y64)
    assert np.all(err <= bound), f"worst excess {np.max(err - bound):.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}"


@pytest.mark.parametrize("name", ["mxfp8_m1", "mxfp8_m5", "mxfp8_m128"])
def test_mxfp8_workloads(name):
    w = synth.WORKLOADS[name]
    _say("mxfp8 workload", name, w)
    inp = synth.gen_workload(name)
    out = run_mxfp8(inp)
    # every output, against both the fp64 and the fp32-sequential oracle
    y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    assert_gate(out, y64, y32, name)


# ---- quantized vocabulary head: W8A16 and the load-time RTN quantizer --------------

W8_CASES = [(m, K, N, G) for m in (1, 3, 5, 8, 16) for (K, N) in ((512, 48), (1280, 32)) for G in (32, 64, 128)]


@pytest.mark.parametrize("M,K,N,G", W8_CASES, ids=["-".join(map(str, c)) for c in W8_CASES])
def test_w8a16_random(M, K, N, G):
    import spec_verify_amd as svq
    _say("w8a16 random M K N G", M, K, N, G)
    inp = synth.gen_w8a16(2000 + 7 * M + K + N + G, M, K, N, G)
    out = svq.w8a16_gemm(dev(inp.x), dev(inp.w), dev(inp.scales), G)
    torch.cuda.synchronize()
    y64, y32 = oracle.w8a16(inp.x, inp.w, inp.scales, G)
    assert_gate(host_bits(out), y64, y32, f"w8a16 M{M} K{K} N{N} G{G}")


@pytest.mark.parametrize("M,K,N,G", [(1, 1024, 32, 128), (5, 1024, 48, 32), (16, 640, 32, 64)])
def test_w8a16_integer_exact(M, K, N, G):
    import spec_verify_amd as svq
    _say("w8a16 intexact M K N G", M, K, N, G)
    inp = synth.gen_w8a16(91 + M, M, K, N, G, kind="intexact")
    out = svq.w8a16_gemm(dev(inp.x), dev(inp.w), dev(inp.scales), G)
    torch.cuda.synchronize()
    xi = oracle.bf16_bits_to_f64(inp.x).astype(np.int64)
    exact = xi @ inp.w.astype(np.int64).T
    np.testing.assert_array_equal(host_bits(out), oracle.bf16_rne(exact.astype(np.float32)))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("N", [80, 77])
def test_rtn_quantize_bit_exact(bits, G, N):
    import spec_verify_amd as svq
    K = 1024   # N = 80 and 77: the last 64-row workgroup holds 16 and 13 rows
    _say("rtn bits G N", bits, G, N)
    wb = synth.gen_dense_bf16(700 + bits + G, N, K)
    wb[3, :G] = 0                                  # an all-zero group: scale 0, codes 0
    q, s = svq.rtn_quantize(dev(wb), bits, G)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.rtn_quantize(wb, bits, G)
    np.testing.assert_array_equal(s.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


def test_rtn_then_gemm_end_to_end():
    import spec_verify_amd as svq
    M, K, N, G = 3, 2560, 512, 128
    _say("rtn -> gemm M K N", M, K, N)
    rng = np.random.default_rng(77)
    x = synth.bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    wb = synth.gen_dense_bf16(78, N, K)
    # int8: codes on the GPU, the W8A16 kernel on them
    q8, s8 = svq.rtn_quantize(dev(wb), 8, G)
    y8 = svq.w8a16_gemm(dev(x), q8, s8, G)
    # int4: GPTQ words on the GPU, repacked, through the W4A16 path
    q4, s4 = svq.rtn_quantize(dev(wb), 4, G)
    y4 = svq.w4a16_gemm(dev(x), svq.q4_repack(q4), s4, N, G)
    torch.cuda.synchronize()
    c8, t8 = oracle.rtn_quantize(wb, 8, G)
    c4, t4 = oracle.rtn_quantize(wb, 4, G)
    np.testing.assert_array_equal(q8.cpu().numpy(), c8)
    np.testing.assert_array_equal(q4.cpu().numpy(), c4)
    assert_gate(host_bits(y8), *oracle.w8a16(x, c8, t8, G), "rtn int8 -> w8a16")
    assert_gate(host_bits(y4), *oracle.w4a16(x, c4, t4, G), "rtn int4 -> w4a16")


@pytest.mark.parametrize("name", ["vocab_w8_m1", "vocab_w4_m1"])
def test_vocab_head_workloads(name):
    import spec_verify_amd as svq
    w = synth.WORKLOADS[name]
    _say("vocab workload", name, w)
    inp = synth.gen_workload(name)
    # every one of the 248320 outputs against the full oracle (about 2.5 GFLOP per
    # sum order: a few seconds on the host)
    if w["op"] == "w8a16":
        out = host_bits(svq.w8a16_gemm(dev(inp.x), dev(inp.w), dev(inp.scales), 128))
        y64, y32 = oracle.w8a16(inp.x, inp.w, inp.scales, 128)
    else:
        out, _ = run_w4a16(inp)
        y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, 128)
    torch.cuda.synchronize()
    assert_gate(out, y64, y32, name)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(out)))


# ---- properties of the launch path -------------------------------------------------

def test_wide_deterministic_and_counters_cleared():
    import spec_verify_amd as svq
    inp = synth.gen_w4a16(5, 128, 2560, 272)
    x, qw, s = dev(inp.x), dev(inp.qweight), dev(inp.scales)
    tiled = svq.q4_repack(qw)
    nbytes = svq.w4a16_workspace_bytes(128, 272, 2560)
    assert nbytes > 0                          # this shape splits tiles across workgroups
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a = svq.w4a16_gemm(x, tiled, s, 272, workspace=ws)
    b = svq.w4a16_gemm(x, tiled, s, 272, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert int(ws[: 256 * 1024].count_nonzero()) == 0   # the arrival counters


def test_dot2_deterministic_and_counters_cleared():
    import spec_verify_amd as svq
    M, K, N = 3, 1280, 5376                    # 336 column blocks
    inp = synth.gen_w4a16(6, M, K, N)
    x, qw, s = dev(inp.x), dev(inp.qweight), dev(inp.scales)
    tiled = svq.q4_repack(qw)
    nbytes = svq.w4a16_workspace_bytes(M, N, K, 128, 1)
    ws = torch.zeros(max(nbytes, 256 * 1024), dtype=torch.uint8, device="cuda")
    a = svq.w4a16_gemm(x, tiled, s, N, kernel=1, workspace=ws)
    b = svq.w4a16_gemm(x, tiled, s, N, kernel=1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert int(ws[: 256 * 1024].count_nonzero()) == 0
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, 128)
    assert_gate(host_bits(a), y64, y32, "dot2 repeated")


# shapes whose K range is split across workgroups, one per kernel family that
# reduces partials through the workspace
SPLIT_CASES = [
    ("w4a16", 2, 5, 5120, 512),     # skinny: 32 column blocks
    ("w4a16", 3, 128, 2560, 512),   # wide: 2 tiles over 20 K steps
    ("mxfp8", 2, 5, 5120, 512),
    ("mxfp8", 3, 128, 2560, 512),
]


@pytest.mark.parametrize("op,kernel,M,K,N", SPLIT_CASES)
def test_split_k_deterministic_and_counters_cleared(op, kernel, M, K, N):
    import spec_verify_amd as svq
    if op == "w4a16":
        inp = synth.gen_w4a16(70 + M, M, K, N)
        x, s = dev(inp.x), dev(inp.scales)
        tiled = svq.q4_repack(dev(inp.qweight))
        nbytes = svq.w4a16_workspace_bytes(M, N, K, 128, kernel)
        run = lambda ws: svq.w4a16_gemm(x, tiled, s, N, 128, kernel=kernel, workspace=ws)
        y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, 128)
    else:
        inp = synth.gen_mxfp8(70 + M, M, K, N)
        x, w, s = dev(inp.x), svq.mxfp8_repack(dev(inp.w)), dev(inp.scales)
        nbytes = svq.mxfp8_workspace_bytes(M, N, K, kernel)
        run = lambda ws: svq.mxfp8_gemm(x, w, s, kernel=kernel, workspace=ws)
        y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    assert nbytes > 256 * 1024                 # counters plus partials: K is split
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = [run(ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))
    assert int(ws[: 256 * 1024].count_nonzero()) == 0   # arrival counters back at zero
    assert_gate(host_bits(outs[0]), y64, y32, f"{op} kernel {kernel} split K")


def test_output_canaries_and_error_path_leave_memory_untouched():
    import spec_verify_amd as svq
    M, K, N = 5, 1024, 64
    inp = synth.gen_w4a16(9, M, K, N)
    x, s = dev(inp.x), dev(inp.scales)
    tiled = svq.q4_repack(dev(inp.qweight))
    guard = 64
    buf = torch.full((M * N + 2 * guard,), 0x7A5A, dtype=torch.int16, device="cuda")
    out = buf[guard:guard + M * N].view(M, N)
    svq.w4a16_gemm(x, tiled, s, N, out=out)
    torch.cuda.synchronize()
    assert int((buf[:guard] != 0x7A5A).sum()) == 0 and int((buf[-guard:] != 0x7A5A).sum()) == 0
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales)
    assert_gate(host_bits(out), y64, y32, "canary run")
    before = buf.clone()
    bad_x = torch.zeros(M * K + 1, dtype=torch.int16, device="cuda")[1:].view(M, K)  # 2-byte offset
    with pytest.raises(svq.SvqError) as e:
        svq.w4a16_gemm(bad_x, tiled, s, N, out=out)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_kernel_names_match_dispatch():
    import spec_verify_amd as svq
    assert svq.w4a16_kernel_name(1, 5120, 5120) == "w4a16_dot2_kernel"
    assert svq.w4a16_kernel_name(1, 1024, 5120) == "w4a16_narrow_kernel"
    assert svq.w4a16_kernel_name(5, 17408, 5120) == "w4a16_skinny_kernel"
    assert svq.w4a16_kernel_name(128, 17408, 5120) == "w4a16_wide_kernel"
