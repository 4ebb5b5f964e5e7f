"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- hand-worked values, closed forms, exact rational brute force, integer
matmul, BLAS, torch's E4M3 decoder, a summation error bound -- so that a dropped
term, a wrong sign, a wrong index or a transposed operand fails at least one.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ---- P6 / P7: element and scale decoders ------------------------------------

def test_e4m3_e8m0_handworked_points():
    n = 0
    for kind, code, value in _rows("e4m3_e8m0_points.txt"):
        c = int(code, 0)
        got = oracle.e4m3_to_f64(c) if kind == "e4m3" else oracle.e8m0_to_f64(c)
        if value == "nan":
            assert math.isnan(got), (kind, code)
        else:
            assert got == float(value), (kind, code, got)
            if value == "-0":
                assert math.copysign(1.0, got) < 0
        n += 1
    assert n >= 20


def test_e4m3_all_codes_closed_form_and_torch():
    torch = pytest.importorskip("torch")
    table = oracle.e4m3_table()
    # closed form from the OCP definition, computed a different way: enumerate
    # (sign, exponent, mantissa) fields explicitly
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            assert math.isnan(table[b])
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert table[b] == (-mag if s else mag), b
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float32).double().numpy()
    finite = ~np.isnan(ref)
    assert finite.sum() == 254
    np.testing.assert_array_equal(table[finite], ref[finite])
    assert np.isnan(table[~finite]).all()


def test_e8m0_all_codes():
    for b in range(255):
        assert oracle.e8m0_to_f64(b) == math.ldexp(1.0, b - 127)
    assert math.isnan(oracle.e8m0_to_f64(255))


def test_fp16_and_bf16_decoders_against_numpy():
    h = np.arange(65536, dtype=np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_to_f64(int(v)) for v in h[::97]])
    r = ref[::97]
    same = (got == r) | (np.isnan(got) & np.isnan(r))
    assert same.all()
    for b in (0x0000, 0x3F80, 0xBF80, 0x4300, 0x0001, 0x7F7F):
        ref = np.array([b], dtype=np.uint32) << 16
        assert oracle.bf16_to_f64(b) == float(ref.view(np.float32)[0])


def test_bf16_rne_ties_and_carries():
    # 257 is halfway between bf16 neighbours 256 and 258 -> ties to even = 256
    # 259 is halfway between 258 and 260 -> ties to even = 260
    vals = np.array([257.0, 259.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -257.0, 0.0], np.float32)
    out = oracle.bf16_rne(vals)
    back = oracle.bf16_bits_to_f64(out)
    np.testing.assert_array_equal(back, [256.0, 260.0, 1.0, 1.0 + 2 ** -6, -256.0, 0.0])
    # against an independent rounding: nearest representable by exhaustive search
    rng = np.random.default_rng(7)
    f = rng.standard_normal(2000).astype(np.float32) * 100
    got = oracle.bf16_bits_to_f64(oracle.bf16_rne(f))
    u = f.view(np.uint32)
    lo = ((u >> 16) << 16).view(np.float32).astype(np.float64)
    hi = (((u >> 16) + 1) << 16).view(np.float32).astype(np.float64)
    fd = f.astype(np.float64)
    dlo, dhi = np.abs(fd - lo), np.abs(hi - fd)
    exp = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(((u >> 16) & 1) == 0, lo, hi)))
    np.testing.assert_array_equal(got, exp)


# ---- P1: GPTQ packing and nibble order --------------------------------------

def test_unpack_roundtrip_and_one_hot_nibbles():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(64, 24), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.q4_unpack(synth.pack_gptq(q)), q)
    for i in range(8):
        word = np.zeros((1, 1), dtype=np.uint32)
        word[0, 0] = 0xB << (4 * i)
        got = oracle.q4_unpack(word.view(np.int32))[:, 0]
        exp = np.zeros(8, dtype=np.uint8)
        exp[i] = 0xB
        np.testing.assert_array_equal(got, exp)


def test_w4a16_handworked_cases():
    for case, word, scale, xpat, expected in _rows("w4a16_handworked.txt"):
        qw = np.array([[int(word, 0)]], dtype=np.uint32).view(np.int32)
        sc = np.array([[int(scale, 0)]], dtype=np.uint16)
        xs = {"ones": [1.0] * 8, "kplus1": [k + 1.0 for k in range(8)],
              "alternating": [1.0, -1.0] * 4}[xpat]
        x = synth.bf16_bits(np.array([xs], dtype=np.float32))
        y64, y32 = oracle.w4a16(x, qw, sc, group_size=8)
        assert y64[0, 0] == float(expected), case
        assert y32[0, 0] == float(expected), case


# ---- P2: identity-scale integer case, exact ---------------------------------

@pytest.mark.parametrize("M,K,N,G", [(3, 256, 48, 128), (5, 384, 32, 64), (2, 128, 16, 32)])
def test_integer_exact_matches_int64_matmul(M, K, N, G):
    inp = synth.gen_w4a16(11 + M, M, K, N, G, kind="intexact", keep_q=True)
    xi = oracle.bf16_bits_to_f64(inp.x).astype(np.int64)
    exact = xi @ (inp.q.astype(np.int64) - 8)           # library integer matmul
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    np.testing.assert_array_equal(y64, exact.astype(np.float64))
    np.testing.assert_array_equal(y32.astype(np.float64), exact.astype(np.float64))


def test_integer_exact_largest_shape_stays_below_2p24():
    # |y| <= 8 * 4 * 17408 = 557056 < 2^24: fp32 accumulation is exact in any order
    assert 8 * 4 * 17408 < 2 ** 24


# ---- P3: exact rational brute force on tiny shapes --------------------------

@pytest.mark.parametrize("M,K,N,G", [(1, 128, 16, 128), (2, 256, 8, 128), (2, 64, 4, 32)])
def test_bruteforce_fraction(M, K, N, G):
    inp = synth.gen_w4a16(5 * K + N, M, K, N, G, keep_q=True)
    y64, _ = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    xf = oracle.bf16_bits_to_f64(inp.x)
    sf = inp.scales.view(np.float16).astype(np.float64)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(xf[m, k])) * (int(inp.q[k, n]) - 8) * Fraction(float(sf[k // G, n]))
            # y64 is the exact sum rounded once per addition in fp64: within K ulps
            assert abs(Fraction(y64[m, n]) - acc) <= Fraction(K) * Fraction(2) ** -52 * (
                sum(abs(Fraction(float(xf[m, k])) * (int(inp.q[k, n]) - 8) * Fraction(float(sf[k // G, n])))
                    for k in range(K)) + 1)


# ---- P4: closed forms that isolate group and nibble indexing ----------------

def test_constant_code_closed_form():
    M, K, N, G = 2, 256, 16, 128
    rng = np.random.default_rng(3)
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    xf = oracle.bf16_bits_to_f64(x)
    s = synth.fp16_bits(rng.uniform(0.002, 0.02, (K // G, N)).astype(np.float32))
    sf = s.view(np.float16).astype(np.float64)
    for c in (0, 3, 8, 15):
        q = np.full((K, N), c, dtype=np.uint8)
        y64, _ = oracle.w4a16(x, synth.pack_gptq(q), s, G)
        xs = xf.reshape(M, K // G, G).sum(axis=2)          # per-group sums of x
        exp = (c - 8) * (xs @ sf)
        np.testing.assert_allclose(y64, exp, rtol=1e-12, atol=1e-12)


def test_one_hot_group_scale_and_single_nibble():
    M, K, N, G = 2, 512, 16, 128
    rng = np.random.default_rng(4)
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    xf = oracle.bf16_bits_to_f64(x)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    for g in range(K // G):
        s = np.zeros((K // G, N), dtype=np.float32)
        s[g, :] = 1.0
        y64, _ = oracle.w4a16(x, synth.pack_gptq(q), synth.fp16_bits(s), G)
        sl = slice(g * G, (g + 1) * G)
        exp = xf[:, sl] @ (q[sl].astype(np.float64) - 8)
        np.testing.assert_allclose(y64, exp, rtol=1e-12, atol=1e-9)
    # one non-8 nibble at (k*, n*): y[:, n*] = x[:, k*] * (q* - 8) * s, all else 0
    q = np.full((K, N), 8, dtype=np.uint8)
    ks, ns, qs = 301, 9, 13
    q[ks, ns] = qs
    s = synth.fp16_bits(np.full((K // G, N), 0.25, dtype=np.float32))
    y64, _ = oracle.w4a16(x, synth.pack_gptq(q), s, G)
    exp = np.zeros((M, N))
    exp[:, ns] = xf[:, ks] * (qs - 8) * 0.25
    np.testing.assert_array_equal(y64, exp)


# ---- P5: dense reduction against BLAS ---------------------------------------

def test_reduction_against_blas():
    M, K, N, G = 4, 1024, 64, 128
    inp = synth.gen_w4a16(9, M, K, N, G, keep_q=True)
    y64, _ = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    xf = oracle.bf16_bits_to_f64(inp.x)
    sf = inp.scales.view(np.float16).astype(np.float64)
    W = (inp.q.astype(np.float64) - 8) * np.repeat(sf, G, axis=0)
    ref = xf @ W
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * rms


def test_fp32_sequential_sum_within_recursive_summation_bound():
    M, K, N, G = 3, 2048, 32, 128
    inp = synth.gen_w4a16(21, M, K, N, G, keep_q=True)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    xf = oracle.bf16_bits_to_f64(inp.x)
    sf = inp.scales.view(np.float16).astype(np.float64)
    W = (inp.q.astype(np.float64) - 8) * np.repeat(sf, G, axis=0)
    absum = np.abs(xf) @ np.abs(W)
    u = 2.0 ** -24
    bound = (K - 1) * u / (1 - (K - 1) * u) * absum
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= bound + 1e-300)
    assert np.any(y32.astype(np.float64) != y64)   # the fp32 mode really rounds


# ---- P8: MXFP8 ---------------------------------------------------------------

def test_mxfp8_integer_exact():
    M, K, N = 3, 256, 16
    inp = synth.gen_mxfp8(31, M, K, N, kind="intexact")
    table = oracle.e4m3_table()
    wi = table[inp.w].astype(np.int64)                  # codes of -8..8 decode exactly
    assert np.all(np.abs(wi) <= 8)
    xi = oracle.bf16_bits_to_f64(inp.x).astype(np.int64)
    exact = xi @ wi.T
    y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    np.testing.assert_array_equal(y64, exact.astype(np.float64))
    np.testing.assert_array_equal(y32.astype(np.float64), exact.astype(np.float64))


def test_mxfp8_block_scale_indexing_closed_form():
    # one block scale raised by 2^3 multiplies exactly that block's contribution by 8
    M, K, N = 2, 128, 8
    inp = synth.gen_mxfp8(32, M, K, N)
    base, _ = oracle.mxfp8(inp.x, inp.w, inp.scales)
    sc = inp.scales.copy()
    n0, b0 = 5, 2
    sc[n0, b0] += 3
    bumped, _ = oracle.mxfp8(inp.x, inp.w, sc)
    table = oracle.e4m3_table()
    xf = oracle.bf16_bits_to_f64(inp.x)
    blk = slice(32 * b0, 32 * b0 + 32)
    contrib = xf[:, blk] @ (table[inp.w[n0, blk]] * 2.0 ** (int(inp.scales[n0, b0]) - 127))
    np.testing.assert_allclose(bumped[:, n0] - base[:, n0], 7 * contrib, rtol=1e-9, atol=1e-12)
    other = [n for n in range(N) if n != n0]
    np.testing.assert_array_equal(bumped[:, other], base[:, other])


def test_mxfp8_against_blas():
    M, K, N = 4, 512, 160
    inp = synth.gen_mxfp8(33, M, K, N)
    y64, _ = oracle.mxfp8(inp.x, inp.w, inp.scales)
    table = oracle.e4m3_table()
    W = table[inp.w] * np.exp2(np.repeat(inp.scales.astype(np.float64) - 127, 32, axis=1))
    ref = oracle.bf16_bits_to_f64(inp.x) @ W.T
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


# ---- P9: invariances ---------------------------------------------------------

def test_power_of_two_scaling_of_x_is_exact():
    inp = synth.gen_w4a16(41, 2, 256, 32, 128)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales)
    x4 = synth.bf16_bits(oracle.bf16_bits_to_f64(inp.x).astype(np.float32) * 4)
    y64b, y32b = oracle.w4a16(x4, inp.qweight, inp.scales)
    np.testing.assert_array_equal(y64b, 4 * y64)
    np.testing.assert_array_equal(y32b, 4 * y32)


def test_group_aligned_k_permutation():
    M, K, N, G = 2, 512, 16, 128
    inp = synth.gen_w4a16(42, M, K, N, G, keep_q=True)
    y64, _ = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    rng = np.random.default_rng(0)
    gperm = rng.permutation(K // G)
    inner = [rng.permutation(G) for _ in range(K // G)]
    perm = np.concatenate([g * G + inner[i] for i, g in enumerate(gperm)])
    xp = inp.x[:, perm]
    qp = inp.q[perm]
    sp = inp.scales[gperm]
    y64p, _ = oracle.w4a16(xp, synth.pack_gptq(qp), sp, G)
    np.testing.assert_allclose(y64p, y64, rtol=0, atol=1e-12 * np.sqrt(np.mean(y64 ** 2)))


# ---- P10: the repack layout -------------------------------------------------

def test_repack_handworked_words():
    N, K = 16, 128
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    q = ((k + n) % 16).astype(np.uint8)
    tiled = oracle.q4_repack(synth.pack_gptq(q)).view(np.uint32)
    cnt = 0
    for lane, j, word in _rows("q4_tile_words.txt"):
        assert tiled[int(lane) * 4 + int(j)] == int(word, 0), (lane, j)
        cnt += 1
    assert cnt == 3


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (160, 1280)])
def test_repack_bijection_and_tile_contents(N, K):
    rng = np.random.default_rng(N + K)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    qw = synth.pack_gptq(q)
    tiled = oracle.q4_repack(qw)
    np.testing.assert_array_equal(oracle.q4_unrepack(tiled, N, K), qw)
    assert tiled.size == K * N // 8
    # independent reading of one random element straight from the layout rule
    slot_of_e = [0, 4, 1, 5, 2, 6, 3, 7]
    t = tiled.view(np.uint32)
    for _ in range(200):
        kk, nn = int(rng.integers(K)), int(rng.integers(N))
        nb, kt, r = nn // 16, kk // 128, kk % 128
        lane = 16 * (r // 32) + nn % 16
        j, e = (r % 32) // 8, r % 8
        word = t[((nb * (K // 128) + kt) * 64 + lane) * 4 + j]
        assert (word >> (4 * slot_of_e[e])) & 15 == q[kk, nn]


# ---- P17: the MXFP8 tile layout ------------------------------------------------

def test_mxfp8_tile_handworked_offsets():
    """Offsets worked by hand from the layout's definition (N = 32, K = 256): a
    matrix whose code encodes its column, and one whose code encodes K, show
    which element each listed offset holds."""
    N, K = 32, 256
    by_col = np.repeat(np.arange(N, dtype=np.uint8)[:, None], K, axis=1)
    by_k = np.repeat(np.arange(K, dtype=np.uint8)[None, :], N, axis=0)
    tc, tk = oracle.mxfp8_tile(by_col), oracle.mxfp8_tile(by_k)
    cnt = 0
    for off, col, k in _rows("mxfp8_tile_bytes.txt"):
        assert (int(tc[int(off)]), int(tk[int(off)])) == (int(col), int(k)), off
        cnt += 1
    assert cnt == 10


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (160, 1280)])
def test_mxfp8_tile_bijection_and_lane_runs(N, K):
    """Every code lands exactly once; untile inverts tile; and read the way a
    kernel lane reads it (two 16-byte loads, one from each 1 KiB half of a
    tile), lane l of tile (nb, kt) gets the 32 consecutive K-elements of column
    16*nb + l%16 that start at 128*kt + 32*(l/16), in order."""
    rng = np.random.default_rng(N * 7 + K)
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    t = oracle.mxfp8_tile(w)
    assert t.size == N * K
    np.testing.assert_array_equal(oracle.mxfp8_untile(t, N, K), w)
    # bijection: the (column, K) labels carried through the layout (column and
    # K split into bytes) come out as a permutation of all N*K pairs
    cols = np.repeat(np.arange(N)[:, None], K, axis=1)
    ks = np.repeat(np.arange(K)[None, :], N, axis=0)
    planes = [oracle.mxfp8_tile(((a >> sh) & 255).astype(np.uint8)).astype(np.int64)
              for a in (cols, ks) for sh in (0, 8)]
    col_of = planes[0] | (planes[1] << 8)
    k_of = planes[2] | (planes[3] << 8)
    assert len(np.unique(col_of * K + k_of)) == N * K
    KT = K // 128
    for _ in range(50):
        nb, kt, lane = int(rng.integers(N // 16)), int(rng.integers(KT)), int(rng.integers(64))
        base = (nb * KT + kt) * 2048
        run = np.concatenate([t[base + 16 * lane: base + 16 * lane + 16],
                              t[base + 1024 + 16 * lane: base + 1024 + 16 * lane + 16]])
        c, k0 = 16 * nb + lane % 16, 128 * kt + 32 * (lane // 16)
        np.testing.assert_array_equal(run, w[c, k0:k0 + 32])
        assert np.all(col_of[base + 16 * lane: base + 16 * lane + 16] == c)


def test_mxfp8_tile_rejects_bad_shapes():
    for N, K in ((8, 128), (16, 64), (16, 200)):
        with pytest.raises(ValueError):
            oracle.mxfp8_tile(np.zeros((N, K), dtype=np.uint8))


def test_gate_accepts_rounding_and_rejects_a_wrong_weight():
    inp = synth.gen_w4a16(51, 1, 5120, 64, 128, keep_q=True)
    y64, _ = oracle.w4a16(inp.x, inp.qweight, inp.scales)
    good = oracle.bf16_rne(y64.astype(np.float32))
    ok, err, rms = oracle.gate(good, y64)
    assert ok and err <= 2 ** -8 * np.max(np.abs(y64))
    bad = oracle.bf16_rne((y64 + 0.05 * rms).astype(np.float32))
    assert not oracle.gate(bad, y64)[0]


# ---- W8A16 (quantized vocabulary head) and its load-time RTN quantizer --------

def _w8_inputs(seed, M, K, N, G, xlo=-4, xhi=5):
    rng = np.random.default_rng(seed)
    x = rng.integers(xlo, xhi, (M, K)).astype(np.float32)
    w = rng.integers(-128, 128, (N, K)).astype(np.int8)
    return synth.bf16_bits(x), w, rng


@pytest.mark.parametrize("M,K,N,G", [(1, 128, 16, 128), (3, 512, 48, 32), (5, 1024, 32, 64)])
def test_w8a16_integer_exact_matches_int64_matmul(M, K, N, G):
    xb, w, _ = _w8_inputs(11 + M, M, K, N, G)
    scales = np.full((K // G, N), 0x3C00, dtype=np.uint16)       # fp16 1.0
    y64, y32 = oracle.w8a16(xb, w, scales, G)
    xi = oracle.bf16_bits_to_f64(xb).astype(np.int64)
    exact = xi @ w.astype(np.int64).T                                # |y| < 2^24: exact in fp32 too
    np.testing.assert_array_equal(y64, exact.astype(np.float64))
    np.testing.assert_array_equal(y32, exact.astype(np.float32))


def test_w8a16_against_blas_and_one_hot_group():
    M, K, N, G = 4, 512, 32, 128
    rng = np.random.default_rng(5)
    xb = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = rng.integers(-128, 128, (N, K)).astype(np.int8)
    s16 = rng.uniform(2e-4, 2e-3, (K // G, N)).astype(np.float16)
    y64, _ = oracle.w8a16(xb, w, s16.view(np.uint16), G)
    deq = w.astype(np.float64) * np.repeat(s16.astype(np.float64).T, G, axis=1)   # [N, K]
    ref = oracle.bf16_bits_to_f64(xb) @ deq.T
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * rms
    # only group 2 has a nonzero scale: y = s * sum over that group's K range
    one = np.zeros((K // G, N), dtype=np.float16)
    one[2, :] = np.float16(0.5)
    y1, _ = oracle.w8a16(xb, w, one.view(np.uint16), G)
    xs = oracle.bf16_bits_to_f64(xb)[:, 2 * G:3 * G]
    np.testing.assert_allclose(y1, 0.5 * xs @ w[:, 2 * G:3 * G].astype(np.float64).T, rtol=0, atol=1e-12 * rms)


def test_rtn_handworked_cases():
    n = 0
    for case, bits, G, sbits, vals, shift, codes in _rows("rtn_handworked.txt"):
        bits, G, shift = int(bits), int(G), int(shift)
        v = np.array([int(t) for t in vals.split(",")], dtype=np.float64) * 2.0 ** shift
        want = np.array([int(t) for t in codes.split(",")], dtype=np.int64)
        wb = synth.bf16_bits(v.astype(np.float32)).reshape(1, -1)
        assert np.array_equal(oracle.bf16_bits_to_f64(wb).ravel(), v), case   # exact in bf16
        q, s = oracle.rtn_quantize(wb, bits, G)
        assert s.shape == (v.size // G, 1) and int(s[0, 0]) == int(sbits, 16), (case, hex(int(s[0, 0])))
        if bits == 8:
            np.testing.assert_array_equal(q.ravel().astype(np.int64), want, err_msg=case)
        else:
            np.testing.assert_array_equal(oracle.q4_unpack(q)[:, 0].astype(np.int64), want + 8, err_msg=case)
        n += 1
    assert n == 5


@pytest.mark.parametrize("bits,G", [(8, 128), (8, 32), (4, 128), (4, 64)])
def test_rtn_error_bound_extremes_and_scaling(bits, G):
    N, K = 24, 512
    rng = np.random.default_rng(40 + bits + G)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wb = synth.bf16_bits(W)
    Wf = oracle.bf16_bits_to_f64(wb)
    q, s = oracle.rtn_quantize(wb, bits, G)
    if bits == 4:
        q = oracle.q4_unpack(q).astype(np.int64).T - 8                 # GPTQ words -> q [N, K]
    q = q.astype(np.int64)
    sf = np.repeat(s.view(np.float16).astype(np.float64).T, G, axis=1)  # [N, K]
    qmax = 2 ** (bits - 1) - 1
    assert q.min() >= -qmax - 1 and q.max() <= qmax
    # round to nearest: every weight within half a step of its code
    assert np.all(np.abs(Wf - q * sf) <= 0.5 * sf * (1 + 2.0 ** -20))
    # the largest |w| of each group lands on +-qmax (the scale is amax / qmax up to fp16 rounding)
    Wg, qg = np.abs(Wf).reshape(N, K // G, G), np.abs(q).reshape(N, K // G, G)
    top = np.take_along_axis(qg, np.argmax(Wg, axis=2)[:, :, None], axis=2)
    assert np.all(top == qmax)
    # a power-of-two factor on the weights moves only the scales
    q2, s2 = oracle.rtn_quantize(synth.bf16_bits(W * np.float32(8.0)), bits, G)
    if bits == 4:
        q2 = oracle.q4_unpack(q2).astype(np.int64).T - 8
    np.testing.assert_array_equal(q2.astype(np.int64), q)
    np.testing.assert_array_equal(s2.view(np.float16).astype(np.float64), 8.0 * s.view(np.float16).astype(np.float64))


def _f32(fr):
    """Nearest binary32 to a Fraction (ties to even), for normal magnitudes."""
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    r = math.floor(m)
    if m - r > Fraction(1, 2) or (m - r == Fraction(1, 2) and r % 2):
        r += 1
    return sgn * r * ulp


def test_rtn_int8_bruteforce_rationals():
    # exact-rational re-derivation on small groups: fp32 quotient rounded by
    # hand, fp16 scale from numpy's own conversion of that fp32 value
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((3, 64)) * 0.05).astype(np.float32)
    wb = synth.bf16_bits(W)
    q, s = oracle.rtn_quantize(wb, 8, 32)
    vals = oracle.bf16_bits_to_f64(wb)
    for n in range(3):
        for g in range(2):
            grp = [Fraction(float(v)) for v in vals[n, 32 * g:32 * g + 32]]
            amax = max(abs(v) for v in grp)
            s32 = _f32(amax / 127)
            s16 = Fraction(float(np.float32(float(s32)).astype(np.float16)))
            assert s16 == Fraction(float(s.view(np.float16)[g, n]))
            for i, v in enumerate(grp):
                r = _f32(v / s16)
                k = math.floor(r)
                if r - k > Fraction(1, 2) or (r - k == Fraction(1, 2) and k % 2):
                    k += 1
                assert int(q[n, 32 * g + i]) == max(-128, min(127, k)), (n, g, i)


# ---- setup-time projection fusion and compressed-tensors ingest ---------------

def _parts4(seed, K, widths, G):
    rng = np.random.default_rng(seed)
    parts = []
    for n in widths:
        q = rng.integers(0, 16, (K, n))
        s = rng.uniform(2e-3, 2e-2, (K // G, n)).astype(np.float16).view(np.uint16)
        parts.append((synth.pack_gptq(q), s))
    return parts


def test_fused_w4_columns_are_the_parts_exactly():
    K, G, widths = 256, 64, [32, 16, 48]
    parts = _parts4(21, K, widths, G)
    wf, sf = oracle.fuse_projections(parts, 4, G)
    assert wf.shape == (K // 8, sum(widths)) and sf.shape == (K // G, sum(widths))
    xb = synth.bf16_bits(np.random.default_rng(22).standard_normal((3, K)).astype(np.float32))
    y64, y32 = oracle.w4a16(xb, wf, sf, G)
    off = 0
    for (w, s), n in zip(parts, widths):
        p64, p32 = oracle.w4a16(xb, w, s, G)
        # each output column is its own sum: fusion changes no bit of it
        np.testing.assert_array_equal(y64[:, off:off + n], p64)
        np.testing.assert_array_equal(y32[:, off:off + n], p32)
        off += n


def test_fused_w8_columns_are_the_parts_exactly():
    K, G, widths = 256, 32, [16, 64]
    rng = np.random.default_rng(23)
    parts = [(rng.integers(-128, 128, (n, K)).astype(np.int8),
              rng.uniform(2e-4, 2e-3, (K // G, n)).astype(np.float16).view(np.uint16)) for n in widths]
    wf, sf = oracle.fuse_projections(parts, 8, G)
    assert wf.shape == (sum(widths), K) and wf.dtype == np.int8
    xb = synth.bf16_bits(rng.standard_normal((2, K)).astype(np.float32))
    y64, _ = oracle.w8a16(xb, wf, sf, G)
    off = 0
    for (w, s), n in zip(parts, widths):
        np.testing.assert_array_equal(y64[:, off:off + n], oracle.w8a16(xb, w, s, G)[0])
        off += n


def test_fused_closed_form_and_tile_layout():
    # part a: every code 1; part b: every code 14 -> words 0x11111111 / 0xeeeeeeee
    K, G = 128, 128
    a = (np.full((K // 8, 16), 0x11111111, dtype=np.uint32).view(np.int32),
         np.full((1, 16), 0x3c00, dtype=np.uint16))
    b = (np.full((K // 8, 32), 0xEEEEEEEE, dtype=np.uint32).view(np.int32),
         np.full((1, 32), 0x4000, dtype=np.uint16))
    wf, sf = oracle.fuse_projections([a, b], 4, G)
    u = wf.view(np.uint32)
    assert np.all(u[:, :16] == 0x11111111) and np.all(u[:, 16:] == 0xEEEEEEEE)
    assert np.all(sf[:, :16] == 0x3c00) and np.all(sf[:, 16:] == 0x4000)
    # x = 1: column sums are K * (q - 8) * s = 128 * -7 * 1 and 128 * 6 * 2
    y64, _ = oracle.w4a16(synth.bf16_bits(np.ones((1, K), np.float32)), wf, sf, G)
    np.testing.assert_array_equal(y64[0], np.r_[np.full(16, -896.0), np.full(32, 1536.0)])
    # the tile layout is column-block-major, so fused tiles are the parts' tiles end to end
    parts = _parts4(24, 256, [16, 48, 32], 128)
    wf, _ = oracle.fuse_projections(parts, 4, 128)
    np.testing.assert_array_equal(oracle.q4_repack(wf),
                                  np.concatenate([oracle.q4_repack(w) for w, _ in parts]))


def test_fuse_rejects_incompatible_projections():
    p = _parts4(25, 256, [16, 32], 64)
    assert oracle.fuse_incompatibility(p, 4, 64) is None
    other_k = _parts4(26, 128, [16], 64)
    assert "different K" in oracle.fuse_incompatibility(p + other_k, 4, 64)
    odd = _parts4(27, 256, [24], 64)
    assert "multiple of 16" in oracle.fuse_incompatibility(p + odd, 4, 64)
    assert "group size" in oracle.fuse_incompatibility(p, 4, 128)     # scales are [K/64, N]
    assert oracle.fuse_incompatibility(p, 5, 64) is not None
    assert oracle.fuse_incompatibility([], 4, 64) is not None
    with pytest.raises(ValueError):
        oracle.fuse_projections(p + odd, 4, 64)


def test_ct_ingest_handworked():
    ct = np.zeros((2, 2), dtype=np.uint32)
    sc = np.zeros((2, 1), dtype=np.uint16)
    gq = np.zeros((2, 2), dtype=np.uint32)
    w = np.full((16, 2), np.nan)
    for row in _rows("ct_handworked.txt"):
        if row[0] == "ct":
            ct[int(row[1]), int(row[2])] = int(row[3], 16)
        elif row[0] == "sc":
            sc[int(row[1]), int(row[2])] = int(row[3], 16)
        elif row[0] == "gptq":
            gq[int(row[1]), int(row[2])] = int(row[3], 16)
        else:
            w[int(row[1]), int(row[2])] = float(row[3])
    assert not np.isnan(w).any()
    qw, s = oracle.ct_to_gptq(ct.view(np.int32), sc)
    np.testing.assert_array_equal(qw.view(np.uint32), gq)
    np.testing.assert_array_equal(s, sc.T)
    deq = (oracle.q4_unpack(qw).astype(np.float64) - 8) * s.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(deq, w)


def test_ct_ingest_gemm_matches_the_ct_definition():
    # dequantize straight from the [N, K/8] words (shifts along the word axis)
    # and multiply with BLAS; the oracle GEMM on the converted tensors must agree
    N, K, G = 48, 512, 128
    rng = np.random.default_rng(28)
    wp = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    ws = rng.uniform(2e-3, 2e-2, (N, K // G)).astype(np.float16)
    q = np.stack([(wp >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], axis=2)   # [N, K/8, 8]
    deq = (q.reshape(N, K).astype(np.float64) - 8) * np.repeat(ws.astype(np.float64), G, axis=1)
    xb = synth.bf16_bits(rng.standard_normal((4, K)).astype(np.float32))
    ref = oracle.bf16_bits_to_f64(xb) @ deq.T
    qw, s = oracle.ct_to_gptq(wp.view(np.int32), ws.view(np.uint16))
    y64, _ = oracle.w4a16(xb, qw, s, G)
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


# ---- MXFP8 quantizer (plain and optimized round-to-nearest) -------------------

def test_e4m3_nearest_against_torch_and_the_generator_encoder():
    torch = pytest.importorskip("torch")
    u = np.arange(0x10000, dtype=np.uint32)
    f = ((u << 16).view(np.float32))
    f = f[np.isfinite(f)]
    a = np.abs(f)
    got = oracle.e4m3_nearest(a)
    inr = a <= 448
    ref = torch.from_numpy(a[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got[inr], ref)
    assert np.all(got[~inr] == 0x7E)
    np.testing.assert_array_equal(got, synth.e4m3_encode_rne(a) & 0x7F)


def test_mxfp8_plain_matches_the_generator_rtn():
    W = (np.random.default_rng(50).standard_normal((8, 512)) * np.float32(0.05)).astype(np.float32)
    W[0, :32] = 0
    W[1, 32:64] *= 1e-30
    wb = synth.bf16_bits(W)
    c, s = oracle.mxfp8_quantize(wb, optimized=False)
    c2, s2 = synth.mxfp8_quantize_rtn(oracle.bf16_bits_to_f64(wb).astype(np.float32))
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(s, s2)


def test_mxfp8_optimized_rtn_handworked_cases():
    n = 0
    for _, name, opt, scale, kept, vals, codes in _rows("mxfp8_optrtn_handworked.txt"):
        v = np.zeros(32, dtype=np.float32)
        vv = [float(t) for t in vals.split(",")]
        v[:len(vv)] = vv
        wb = synth.bf16_bits(v).reshape(1, 32)
        assert np.array_equal(oracle.bf16_bits_to_f64(wb).ravel(), v.astype(np.float64)), name
        c, s, ch = oracle.mxfp8_quantize(wb, optimized=bool(int(opt)), return_choice=True)
        want = np.zeros(32, dtype=np.uint8)
        cc = [int(t, 16) for t in codes.split(",")]
        want[:len(cc)] = cc
        assert int(s[0, 0]) == int(scale) and int(ch[0, 0]) == int(kept), name
        np.testing.assert_array_equal(c[0], want, err_msg=name)
        n += 1
    assert n == 8


def _exact_block(vals, b):
    """Exact rational E4M3 codes and squared error of one block at E8M0 code b:
    every finite magnitude is scanned, ties go to the even code."""
    mags = [Fraction(oracle.e4m3_to_f64(c)) for c in range(0x7F)]
    scale = Fraction(2) ** (b - 127)
    codes, err = [], Fraction(0)
    for v in vals:
        a = abs(v) / scale
        best = None
        for c, m in enumerate(mags):
            d = abs(a - m)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        c = best[1]
        dec = mags[c] * scale * (-1 if v < 0 else 1)
        codes.append(c | (0x80 if v < 0 else 0))
        err += (v - dec) ** 2
    return codes, err


def test_mxfp8_optimized_rtn_exact_rational_bruteforce():
    rng = np.random.default_rng(51)
    W = (rng.standard_normal((2, 8 * 32)) * 0.03).astype(np.float32)
    # force a few blocks to saturate at the baseline scale: amax / 2^X0 in (448, 512)
    for blk in (1, 4, 6, 9, 13):
        r, k = divmod(blk, 8)
        seg = W[r, 32 * k:32 * k + 32]
        X0 = math.floor(math.log2(float(np.abs(seg).max()))) - 8
        seg[int(np.argmax(np.abs(seg)))] = np.float32(rng.uniform(452, 510) * 2.0 ** X0)
    wb = synth.bf16_bits(W)
    c, s, ch = oracle.mxfp8_quantize(wb, optimized=True, return_choice=True)
    vals = oracle.bf16_bits_to_f64(wb)
    chosen = 0
    for r in range(2):
        for k in range(8):
            blk = [Fraction(float(t)) for t in vals[r, 32 * k:32 * k + 32]]
            amax = max(abs(t) for t in blk)
            b0 = min(max(math.floor(math.log2(amax)) - 8 + 127, 0), 254)
            cands = [_exact_block(blk, b) for b in (b0, b0 + 1, b0 - 1)]
            i = int(ch[r, k])
            best = min(e for _, e in cands)
            # the kept candidate is the exact minimum, up to fp32 rounding of the sums
            assert cands[i][1] <= best * (1 + Fraction(1, 10 ** 6)), (r, k, i)
            assert int(s[r, k]) == (b0, b0 + 1, b0 - 1)[i]
            assert list(c[r, 32 * k:32 * k + 32]) == cands[i][0], (r, k)
            chosen += i == 1
    assert chosen >= 4


def test_mxfp8_optimized_rtn_invariants():
    rng = np.random.default_rng(52)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    wb = synth.bf16_bits(W)
    cp, sp = oracle.mxfp8_quantize(wb, optimized=False)
    co, so, ch = oracle.mxfp8_quantize(wb, optimized=True, return_choice=True)
    tab = oracle.e4m3_table()
    Wf = oracle.bf16_bits_to_f64(wb).reshape(64, 32, 32)

    def blk_err(c, s):
        d = tab[c].reshape(64, 32, 32) * np.ldexp(1.0, s.astype(np.int64) - 127)[:, :, None]
        return ((Wf - d) ** 2).sum(axis=2)
    ep, eo = blk_err(cp, sp), blk_err(co, so)
    assert np.all(eo <= ep * (1 + 1e-6))
    # half the baseline scale saturates the block maximum, so it is never kept
    assert not np.any(ch == 2)
    # twice the scale is kept only where the baseline saturates an element
    X0 = sp.astype(np.int64) - 127
    sat = np.abs(Wf).max(axis=2) / np.ldexp(1.0, X0) > 448
    assert np.all(sat[ch == 1]) and np.any(ch == 1)
    np.testing.assert_array_equal(so, np.where(ch == 1, sp + 1, sp))
    # a power-of-two factor moves only the scales
    c8, s8 = oracle.mxfp8_quantize(synth.bf16_bits(W * np.float32(2.0 ** 5)), optimized=True)
    np.testing.assert_array_equal(c8, co)
    np.testing.assert_array_equal(s8.astype(np.int64), so.astype(np.int64) + 5)


# ---- point evaluators: the sampled-output forms the full-size checks rely on ----

def _points(M, N, n, seed):
    """Random (row, col) pairs plus the four corners and repeated points."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, M, n)
    cols = rng.integers(0, N, n)
    rows = np.concatenate([[0, M - 1, 0, M - 1], rows, rows[:3]])
    cols = np.concatenate([[0, 0, N - 1, N - 1], cols, cols[:3]])
    return rows, cols


@pytest.mark.parametrize("G", [32, 64, 128])
def test_w4a16_points_are_the_full_result(G):
    M, K, N = 5, 512, 48
    inp = synth.gen_w4a16(61 + G, M, K, N, G)
    y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
    rows, cols = _points(M, N, 40, G)
    p64, p32 = oracle.w4a16_points(inp.x, inp.qweight, inp.scales, G, rows, cols)
    np.testing.assert_array_equal(p64.view(np.uint64), y64[rows, cols].view(np.uint64))
    np.testing.assert_array_equal(p32.view(np.uint32), y32[rows, cols].view(np.uint32))


def test_w4a16_points_integer_exact_against_int64_matmul():
    M, K, N, G = 3, 384, 32, 64
    inp = synth.gen_w4a16(67, M, K, N, G, kind="intexact", keep_q=True)
    exact = oracle.bf16_bits_to_f64(inp.x).astype(np.int64) @ (inp.q.astype(np.int64) - 8)
    rows, cols = _points(M, N, 30, 5)
    p64, p32 = oracle.w4a16_points(inp.x, inp.qweight, inp.scales, G, rows, cols)
    np.testing.assert_array_equal(p64, exact[rows, cols].astype(np.float64))
    np.testing.assert_array_equal(p32.astype(np.float64), exact[rows, cols].astype(np.float64))


def test_mxfp8_points_are_the_full_result():
    M, K, N = 4, 512, 144
    inp = synth.gen_mxfp8(71, M, K, N)
    y64, y32 = oracle.mxfp8(inp.x, inp.w, inp.scales)
    rows, cols = _points(M, N, 40, 7)
    p64, p32 = oracle.mxfp8_points(inp.x, inp.w, inp.scales, rows, cols)
    np.testing.assert_array_equal(p64.view(np.uint64), y64[rows, cols].view(np.uint64))
    np.testing.assert_array_equal(p32.view(np.uint32), y32[rows, cols].view(np.uint32))
    # integer-valued inputs: the points equal an int64 matmul of the decoded codes
    ie = synth.gen_mxfp8(72, M, K, N, kind="intexact")
    exact = oracle.bf16_bits_to_f64(ie.x).astype(np.int64) @ oracle.e4m3_table()[ie.w].astype(np.int64).T
    q64, q32 = oracle.mxfp8_points(ie.x, ie.w, ie.scales, rows, cols)
    np.testing.assert_array_equal(q64, exact[rows, cols].astype(np.float64))
    np.testing.assert_array_equal(q32.astype(np.float64), exact[rows, cols].astype(np.float64))


@pytest.mark.parametrize("G", [32, 64, 128])
def test_w8a16_points_are_the_full_result(G):
    M, K, N = 3, 512, 48
    inp = synth.gen_w8a16(81 + G, M, K, N, G)
    y64, y32 = oracle.w8a16(inp.x, inp.w, inp.scales, G)
    rows, cols = _points(M, N, 40, 8 + G)
    p64, p32 = oracle.w8a16_points(inp.x, inp.w, inp.scales, G, rows, cols)
    np.testing.assert_array_equal(p64.view(np.uint64), y64[rows, cols].view(np.uint64))
    np.testing.assert_array_equal(p32.view(np.uint32), y32[rows, cols].view(np.uint32))
    ie = synth.gen_w8a16(82 + G, M, K, N, G, kind="intexact")
    exact = oracle.bf16_bits_to_f64(ie.x).astype(np.int64) @ ie.w.astype(np.int64).T
    q64, _ = oracle.w8a16_points(ie.x, ie.w, ie.scales, G, rows, cols)
    np.testing.assert_array_equal(q64, exact[rows, cols].astype(np.float64))


def test_points_reject_out_of_range_indices():
    inp = synth.gen_w4a16(91, 2, 256, 32, 128)
    mx = synth.gen_mxfp8(92, 2, 256, 32)
    w8 = synth.gen_w8a16(93, 2, 256, 32, 128)
    for rows, cols in (([2], [0]), ([0], [32]), ([-1], [0]), ([0], [-1])):
        with pytest.raises(ValueError):
            oracle.w4a16_points(inp.x, inp.qweight, inp.scales, 128, rows, cols)
        with pytest.raises(ValueError):
            oracle.mxfp8_points(mx.x, mx.w, mx.scales, rows, cols)
        with pytest.raises(ValueError):
            oracle.w8a16_points(w8.x, w8.w, w8.scales, 128, rows, cols)
