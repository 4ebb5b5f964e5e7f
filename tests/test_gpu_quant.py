"""GPU parity of the MXFP8 quantizer (plain and optimized round-to-nearest)
through the C ABI: codes and scales bit for bit against the oracle, on random
weights, on blocks built to hit every branch (saturation, zeros, signed zeros,
fp32-subnormal scores, bf16 subnormals, the largest bf16 values, every finite
bf16 pattern), on ragged shapes, and on sampled rows of a full-size projection;
then quantize -> MXFP8 GEMM against the oracle GEMM.
"""
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
    import os
    import spec_verify_amd as svq
    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    svq.lib()
    yield


def _say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def _quant(wb, optimized):
    import spec_verify_amd as svq
    w = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16)).cuda()
    c, s = svq.mxfp8_quantize(w, optimized)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _check(wb, optimized, label):
    c, s = _quant(wb, optimized)
    c_ref, s_ref = oracle.mxfp8_quantize(wb, optimized)
    np.testing.assert_array_equal(s, s_ref, err_msg=f"{label} scales")
    np.testing.assert_array_equal(c, c_ref, err_msg=f"{label} codes")
    return c, s


@pytest.mark.parametrize("optimized", [True, False])
@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (128, 512), (77, 1056)])
def test_mxfp8_quantize_random(N, K, optimized):
    _say("mxfp8 quantize", N, K, optimized)
    W = (np.random.default_rng(N + K).standard_normal((N, K)) * 0.02).astype(np.float32)
    _check(synth.bf16_bits(W), optimized, f"{N}x{K}")


def _crafted():
    rng = np.random.default_rng(60)
    blocks = []
    base = (rng.standard_normal((40, 32)) * 0.02).astype(np.float32)
    for i in range(40):                          # baseline saturates the maximum
        b = base[i].copy()
        j = int(np.argmax(np.abs(b)))
        X0 = np.floor(np.log2(np.abs(b[j]))) - 8
        b[j] = np.float32(np.sign(b[j]) * rng.uniform(449, 511) * 2.0 ** X0)
        blocks.append(b)
    blocks.append(np.zeros(32, np.float32))
    blocks.append(np.full(32, -0.0, np.float32))
    z = np.zeros(32, np.float32)
    z[3], z[7] = 1.0, -2.0 ** -20
    blocks.append(z)
    blocks.append((rng.standard_normal(32) * 2.0 ** -60).astype(np.float32))    # scores in fp32 subnormals
    blocks.append((rng.standard_normal(32) * 2.0 ** -128).astype(np.float32))   # bf16 subnormals, E8M0 clamp
    blocks.append((rng.uniform(-1, 1, 32) * 3.0e38).astype(np.float32))         # near the bf16 maximum
    t = np.zeros(32, np.float32)
    t[0], t[1] = 452.0, 2.0 ** -9                                                # x2 costs a subnormal step
    blocks.append(t)
    wb = synth.bf16_bits(np.stack(blocks))
    # every finite bf16 pattern, shuffled into blocks
    u = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    f = (u.astype(np.uint32) << 16).view(np.float32)
    u = u[np.isfinite(f)]
    u = rng.permutation(u)
    u = u[:u.size // 32 * 32].reshape(-1, 32)
    return np.concatenate([wb.reshape(-1, 32), u])          # [2087, 32]: one block per row


@pytest.mark.parametrize("optimized", [True, False])
def test_mxfp8_quantize_crafted_blocks(optimized):
    wb = _crafted()
    c, s = _check(wb, optimized, "crafted")
    if optimized:
        cp, sp = oracle.mxfp8_quantize(wb, False)
        assert np.any(s != sp)                  # the doubled scale is taken somewhere


def test_mxfp8_quantize_full_size_sampled_rows():
    # one MLP-sized projection [17408, 5120]: each row is quantized on its own,
    # so sampled rows of the device result are checked against the oracle
    N, K = 17408, 5120
    wb = synth.gen_dense_bf16(970, N, K)
    c, s = _quant(wb, True)
    rows = np.random.default_rng(7).choice(N, 96, replace=False)
    c_ref, s_ref = oracle.mxfp8_quantize(wb[rows], True)
    np.testing.assert_array_equal(s[rows], s_ref)
    np.testing.assert_array_equal(c[rows], c_ref)


def test_mxfp8_quantize_then_gemm():
    import spec_verify_amd as svq
    N, K, M = 256, 1024, 5
    wb = synth.gen_dense_bf16(971, N, K, std=0.05)
    w = torch.from_numpy(wb.view(np.int16)).cuda()
    c, s = svq.mxfp8_quantize(w, True)
    x = synth.gen_w4a16(972, M, K, 16).x
    out = svq.mxfp8_gemm(torch.from_numpy(x.view(np.int16)).cuda(), svq.mxfp8_repack(c), s)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mxfp8_quantize(wb, True)
    y64, y32 = oracle.mxfp8(x, c_ref, s_ref)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ok64, e64, rms = oracle.gate(got, y64)
    ok32, e32, _ = oracle.gate(got, y32.astype(np.float64))
    assert ok64 and ok32, (e64, e32, rms)
