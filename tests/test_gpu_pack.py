"""GPU parity of the setup-time layout steps through the C ABI: projection
fusion (one launch that concatenates projections along N and repacks them) and
the compressed-tensors ingest (a transpose of words and scales). Layout results
are compared bit for bit with the oracle; GEMMs on fused or ingested weights
go through the same parity gate as every other GEMM (max |fp32(out) - y_ref|
<= 2e-2 * RMS(y_ref) against the fp64 and the fp32-sequential oracle), or bit
for bit on integer-valued inputs.
"""
import sys
import warnings

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


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_gate(out, y64, y32, label):
    ok64, e64, rms = oracle.gate(out, y64)
    ok32, e32, _ = oracle.gate(out, y32.astype(np.float64))
    assert ok64 and ok32, f"{label}: err64={e64:.4g} err32={e32:.4g} rms={rms:.4g}"


# ---- fusion: layout ----------------------------------------------------------------

FUSE_CASES = [
    (4, 128, 128, [16]),                       # one part: the plain repack
    (4, 256, 64, [16, 48, 32]),
    (4, 384, 32, [32] * 16),                   # the most parts one call takes
    (4, 5120, 128, [1024, 1024, 6144]),        # K/V/Q
    (8, 256, 32, [16, 64]),
    (8, 5120, 128, [1024, 1024, 6144]),
]


@pytest.mark.parametrize("bits,K,G,widths", FUSE_CASES,
                         ids=[f"int{b}-K{k}-G{g}-{len(w)}parts" for b, k, g, w in FUSE_CASES])
def test_fuse_bit_exact(bits, K, G, widths):
    import spec_verify_amd as svq
    _say("fuse", bits, K, G, widths)
    inp = synth.gen_fusion(800 + K + len(widths), 1, K, widths, G, bits)
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, bits, G)
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    wf, sf = svq.fuse_projections(parts, bits, G)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(sf), sf_ref)
    if bits == 4:
        np.testing.assert_array_equal(wf.cpu().numpy(), oracle.q4_repack(wf_ref))
    else:
        np.testing.assert_array_equal(wf.cpu().numpy(), wf_ref)


def test_fuse_writes_exactly_its_outputs():
    # canaries around both outputs stay untouched
    import spec_verify_amd as svq
    K, G, widths = 256, 64, [16, 32]
    inp = synth.gen_fusion(811, 1, K, widths, G, 4)
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    Nt = sum(widths)
    wbuf = torch.full((K * Nt // 8 + 128,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    sbuf = torch.full(((K // G) * Nt + 256,), 0x3A3A, dtype=torch.int16, device="cuda")
    svq.fuse_projections(parts, 4, G, weight_fused=wbuf[64:64 + K * Nt // 8],
                         scales_fused=sbuf[128:128 + (K // G) * Nt].view(torch.float16))
    torch.cuda.synchronize()
    w = wbuf.cpu().numpy()
    s = sbuf.cpu().numpy()
    assert np.all(w[:64] == 0x5A5A5A5A) and np.all(w[64 + K * Nt // 8:] == 0x5A5A5A5A)
    assert np.all(s[:128] == 0x3A3A) and np.all(s[128 + (K // G) * Nt:] == 0x3A3A)
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 4, G)
    np.testing.assert_array_equal(w[64:64 + K * Nt // 8], oracle.q4_repack(wf_ref))
    np.testing.assert_array_equal(s[128:128 + (K // G) * Nt].view(np.uint16), sf_ref.ravel())


def test_fuse_or_keep_leaves_incompatible_projections_alone():
    import spec_verify_amd as svq
    a = synth.gen_fusion(812, 1, 256, [16], 64, 4).parts[0]
    b = synth.gen_fusion(813, 1, 128, [16], 64, 4).parts[0]        # another K
    c = synth.gen_fusion(814, 1, 256, [24], 64, 4).parts[0]        # width not a multiple of 16
    for other in (b, c):
        parts = [(dev(a[0]), dev(a[1])), (dev(other[0]), dev(other[1]))]
        with warnings.catch_warnings(record=True) as rec:
            warnings.simplefilter("always")
            assert svq.fuse_or_keep(parts, 4, 64) is None
        assert any("not fused" in str(r.message) for r in rec)


# ---- fusion: GEMMs on fused weights --------------------------------------------------

@pytest.mark.parametrize("M,kernel", [(1, 0), (5, 0), (5, 1), (40, 0)])
def test_fused_w4a16_gemm(M, kernel):
    import spec_verify_amd as svq
    K, G, widths = 1024, 128, [256, 128, 640]
    _say("fused gemm", M, kernel)
    inp = synth.gen_fusion(820 + M, M, K, widths, G, 4)
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 4, G)
    y64, y32 = oracle.w4a16(inp.x, wf_ref, sf_ref, G)
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    wf, sf = svq.fuse_projections(parts, 4, G)
    out = svq.w4a16_gemm(dev(inp.x), wf, sf, sum(widths), G, kernel=kernel)
    torch.cuda.synchronize()
    assert_gate(host_u16(out), y64, y32, f"fused M={M}")


def test_fused_w4a16_integer_exact_equals_parts():
    # integer-valued inputs: the fused GEMM's columns equal the separate GEMMs' bits
    import spec_verify_amd as svq
    K, G, widths = 640, 64, [48, 16, 96]
    inp = synth.gen_fusion(830, 3, K, widths, G, 4, kind="intexact")
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    x = dev(inp.x)
    wf, sf = svq.fuse_projections(parts, 4, G)
    yf = host_u16(svq.w4a16_gemm(x, wf, sf, sum(widths), G))
    off = 0
    for (w, s), n in zip(parts, widths):
        yp = host_u16(svq.w4a16_gemm(x, svq.q4_repack(w), s, n, G))
        np.testing.assert_array_equal(yf[:, off:off + n], yp)
        off += n
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 4, G)
    y64, _ = oracle.w4a16(inp.x, wf_ref, sf_ref, G)
    np.testing.assert_array_equal(yf, oracle.bf16_rne(y64.astype(np.float32)))


def test_fused_w8a16_gemm():
    import spec_verify_amd as svq
    K, G, widths = 1024, 128, [64, 192]
    inp = synth.gen_fusion(840, 2, K, widths, G, 8)
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 8, G)
    y64, y32 = oracle.w8a16(inp.x, wf_ref, sf_ref, G)
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    wf, sf = svq.fuse_projections(parts, 8, G)
    out = svq.w8a16_gemm(dev(inp.x), wf, sf, G)
    torch.cuda.synchronize()
    assert_gate(host_u16(out), y64, y32, "fused w8a16")


@pytest.mark.parametrize("name", sorted(synth.FUSIONS))
def test_fusion_workloads_sampled(name):
    # full-size K/V/Q and gate/up fusion in the benchmark's launch configuration
    import spec_verify_amd as svq
    f = synth.FUSIONS[name]
    _say("fusion workload", name)
    inp = synth.gen_fusion(f["seed"], f["M"], f["K"], f["widths"], 128, 4)
    wf_ref, sf_ref = oracle.fuse_projections(inp.parts, 4, 128)
    parts = [(dev(w), dev(s)) for w, s in inp.parts]
    wf, sf = svq.fuse_projections(parts, 4, 128)
    Nt = sum(f["widths"])
    out = svq.w4a16_gemm(dev(inp.x), wf, sf, Nt, 128)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = rng.integers(0, f["M"], 384)
    cols = np.r_[rng.integers(0, Nt, 376), np.cumsum([0] + f["widths"][:-1]), Nt - 1]
    rows = rows[:cols.size]
    y64, y32 = oracle.w4a16_points(inp.x, wf_ref, sf_ref, 128, rows, cols)
    got = host_u16(out)[rows, cols]
    assert_gate(got, y64, y32, name)
    # the fused tiles are the oracle's repack of the concatenation (sampled words)
    idx = rng.integers(0, wf.numel(), 4096)
    np.testing.assert_array_equal(wf.cpu().numpy()[idx], oracle.q4_repack(wf_ref)[idx])


# ---- compressed-tensors ingest -----------------------------------------------------------

CT_CASES = [(1, 32, 32), (100, 96, 32), (16, 128, 128), (257, 640, 64), (5120, 5120, 128),
            (17408, 5120, 128)]


@pytest.mark.parametrize("N,K,G", CT_CASES, ids=[f"N{n}-K{k}-G{g}" for n, k, g in CT_CASES])
def test_ct_to_gptq_bit_exact(N, K, G):
    import spec_verify_amd as svq
    _say("ct ingest", N, K, G)
    wp, ws = synth.gen_ct_w4a16(900 + N, N, K, G)
    qw_ref, s_ref = oracle.ct_to_gptq(wp, ws)
    qw, s = svq.ct_to_gptq(dev(wp), dev(ws), G)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qw.cpu().numpy(), qw_ref)
    np.testing.assert_array_equal(host_u16(s), s_ref)


def test_ct_ingest_end_to_end_gemm():
    # compressed-tensors tensors -> GPTQ -> repack -> GEMM, against the oracle GEMM
    # on the oracle's own ingest
    import spec_verify_amd as svq
    N, K, G, M = 512, 2048, 64, 5
    wp, ws = synth.gen_ct_w4a16(950, N, K, G)
    x = synth.gen_w4a16(951, M, K, 16, G).x
    qw_ref, s_ref = oracle.ct_to_gptq(wp, ws)
    y64, y32 = oracle.w4a16(x, qw_ref, s_ref, G)
    qw, s = svq.ct_to_gptq(dev(wp), dev(ws), G)
    out = svq.w4a16_gemm(dev(x), svq.q4_repack(qw), s, N, G)
    torch.cuda.synchronize()
    assert_gate(host_u16(out), y64, y32, "ct end to end")
