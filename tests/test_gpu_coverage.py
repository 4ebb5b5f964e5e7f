"""GPU coverage of the launch paths through the C ABI: the automatic kernel choice
over a sweep of M, the shortest K every kernel accepts, output tiles shared by
several workgroups of the wide kernels (their fp32 partials summed by a second
launch), guard bytes around the workspace and the output, and the probes.

Every result is compared with the CPU oracle (fp64 and fp32-sequential sums)
under the parity gate max|err| <= 2e-2 * RMS(ref); repeated runs must also be
bit-identical, since all reductions run in a fixed order.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

COUNTER_BYTES = 256 * 1024


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


def assert_gate(out, y64, y32, label):
    ok64, e64, rms = oracle.gate(out, y64)
    ok32, e32, _ = oracle.gate(out, y32.astype(np.float64))
    assert ok64 and ok32, f"{label}: err64={e64:.4g} err32={e32:.4g} rms={rms:.4g}"


class W4:
    """A W4A16 problem on the device, with its oracle result."""

    def __init__(self, seed, M, K, N, G):
        import spec_verify_amd as svq
        self.inp = synth.gen_w4a16(seed, M, K, N, G)
        self.M, self.K, self.N, self.G = M, K, N, G
        self.x, self.s = dev(self.inp.x), dev(self.inp.scales)
        self.tiled = svq.q4_repack(dev(self.inp.qweight))

    def ref(self):
        return oracle.w4a16(self.inp.x, self.inp.qweight, self.inp.scales, self.G)

    def run(self, kernel=0, out=None, workspace=None):
        import spec_verify_amd as svq
        return svq.w4a16_gemm(self.x, self.tiled, self.s, self.N, self.G, out=out, kernel=kernel,
                              workspace=workspace)

    def ws_bytes(self, kernel=0):
        import spec_verify_amd as svq
        return svq.w4a16_workspace_bytes(self.M, self.N, self.K, self.G, kernel)


class MX:
    def __init__(self, seed, M, K, N):
        self.inp = synth.gen_mxfp8(seed, M, K, N)
        self.M, self.K, self.N = M, K, N
        import spec_verify_amd as svq
        self.x, self.w, self.s = dev(self.inp.x), svq.mxfp8_repack(dev(self.inp.w)), dev(self.inp.scales)

    def ref(self):
        return oracle.mxfp8(self.inp.x, self.inp.w, self.inp.scales)

    def run(self, kernel=0, out=None, workspace=None):
        import spec_verify_amd as svq
        return svq.mxfp8_gemm(self.x, self.w, self.s, out=out, kernel=kernel, workspace=workspace)

    def ws_bytes(self, kernel=0):
        import spec_verify_amd as svq
        return svq.mxfp8_workspace_bytes(self.M, self.N, self.K, kernel)


# ---- the automatic kernel choice over M ---------------------------------------------

SWEEP_M = list(range(1, 18)) + [31, 32, 33, 127, 128, 129]


@pytest.mark.parametrize("M", SWEEP_M)
def test_auto_dispatch_w4a16_m_sweep(M):
    import spec_verify_amd as svq
    G = (32, 64, 128)[M % 3]
    K, N = 1280, 384
    _say("auto w4a16 M K N G", M, K, N, G)
    p = W4(5000 + M, M, K, N, G)
    want = {1: "w4a16_dot2_kernel"}.get(M, "w4a16_skinny_kernel" if M <= 16 else "w4a16_wide_kernel")
    assert svq.w4a16_kernel_name(M, N, K, G) == want
    assert svq.kernel_name(svq.OP_W4A16, M, N, K, G) == want
    out = p.run()
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *p.ref(), f"auto w4a16 M{M}")


@pytest.mark.parametrize("M", SWEEP_M)
def test_auto_dispatch_mxfp8_m_sweep(M):
    import spec_verify_amd as svq
    K, N = 1280, 256
    _say("auto mxfp8 M K N", M, K, N)
    p = MX(5100 + M, M, K, N)
    want = "mxfp8_dot2_kernel" if M <= 2 else ("mxfp8_skinny_kernel" if M <= 16 else "mxfp8_wide_kernel")
    assert svq.mxfp8_kernel_name(M, N, K) == want
    out = p.run()
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *p.ref(), f"auto mxfp8 M{M}")


# ---- the shortest K: one and two 128-row tiles, on every kernel ----------------------

SMALL_K_W4 = (
    [("dot2", 1, m, N, G) for m in (1, 3, 8) for N in (48,) for G in (32, 64, 128)]
    + [("narrow", 1, m, 1024, G) for m in (1, 2) for G in (32, 128)]
    + [("skinny", 2, m, 48, G) for m in (2, 5, 8, 16) for G in (32, 64, 128)]
    + [("wide", 3, m, 272, G) for m in (17, 128) for G in (32, 64, 128)]
)


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("name,kernel,M,N,G", SMALL_K_W4, ids=["-".join(map(str, c)) for c in SMALL_K_W4])
def test_w4a16_smallest_k(K, name, kernel, M, N, G):
    import spec_verify_amd as svq
    _say("small K w4a16", name, "M K N G", M, K, N, G)
    if name == "narrow":
        if torch.cuda.get_device_properties(0).multi_processor_count != 256:
            pytest.skip("narrow-unit shape chosen for a 256-CU part")
        assert svq.w4a16_kernel_name(M, N, K, G, kernel=1) == "w4a16_narrow_kernel"
    p = W4(5200 + K + M + N + G, M, K, N, G)
    out = p.run(kernel)
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *p.ref(), f"{name} M{M} K{K} N{N} G{G}")


SMALL_K_MX = [("dot2", 1, 1, 128), ("dot2", 1, 5, 256), ("skinny", 2, 5, 128), ("skinny", 2, 16, 256),
              ("wide", 3, 17, 128), ("wide", 3, 128, 256)]


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("name,kernel,M,N", SMALL_K_MX, ids=["-".join(map(str, c)) for c in SMALL_K_MX])
def test_mxfp8_smallest_k(K, name, kernel, M, N):
    _say("small K mxfp8", name, "M K N", M, K, N)
    p = MX(5300 + K + M + N, M, K, N)
    out = p.run(kernel)
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *p.ref(), f"mxfp8 {name} M{M} K{K} N{N}")


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("M,G", [(1, 128), (5, 32), (16, 64)])
def test_w8a16_smallest_k(K, M, G):
    import spec_verify_amd as svq
    N = 48
    _say("small K w8a16 M K N G", M, K, N, G)
    inp = synth.gen_w8a16(5400 + K + M + G, M, K, N, G)
    out = svq.w8a16_gemm(dev(inp.x), dev(inp.w), dev(inp.scales), G)
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *oracle.w8a16(inp.x, inp.w, inp.scales, G), f"w8a16 M{M} K{K} G{G}")


# ---- shared tiles of the wide kernels: partials summed by a second launch ------------

# W4A16 wide shapes (128 x 256 tiles) whose tiles are shared: 2 tiles over 20 K
# steps; one tile over 40 K steps (40 contributors, summed in groups of 8) at
# G = 32 and with a ragged last row tile; two row tiles with stream-K ranges that
# cross tiles (more tiles than CUs: each workgroup holds partials of two tiles).
W4_SHARED = [(128, 2560, 272, 128), (64, 5120, 256, 32), (100, 5120, 256, 128), (256, 640, 40960, 64)]


@pytest.mark.parametrize("M,K,N,G", W4_SHARED, ids=["-".join(map(str, c)) for c in W4_SHARED])
def test_w4a16_wide_shared_tiles_second_launch(M, K, N, G):
    _say("w4a16 wide shared M K N G", M, K, N, G)
    p = W4(5550 + M + K + N + G, M, K, N, G)
    nbytes = p.ws_bytes(3)
    assert nbytes > COUNTER_BYTES                # tiles are shared: partials exist
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = [p.run(3, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    assert_gate(host_bits(outs[0]), *p.ref(), f"w4a16 wide shared M{M} K{K} N{N}")


# MXFP8 wide shapes whose tiles are shared: the partials are summed by a second
# launch in contributor order. 128 x 2560 x 272: 3 column tiles over 20 K steps;
# 64 x 5120 x 256: 2 tiles over 40 K steps, 40 contributors each (the sum runs in
# groups of 8); 200 x 1280 x 640: 2 row tiles x 5 column tiles.
MX_SHARED = [(128, 2560, 272), (64, 5120, 256), (200, 1280, 640), (17, 5120, 128)]


@pytest.mark.parametrize("M,K,N", MX_SHARED, ids=["-".join(map(str, c)) for c in MX_SHARED])
def test_mxfp8_wide_shared_tiles_second_launch(M, K, N):
    _say("mxfp8 wide shared M K N", M, K, N)
    p = MX(5650 + M + K + N, M, K, N)
    nbytes = p.ws_bytes(3)
    assert nbytes > COUNTER_BYTES                # tiles are shared: partials exist
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = [p.run(3, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    assert_gate(host_bits(outs[0]), *p.ref(), f"mxfp8 wide shared M{M} K{K} N{N}")


# ---- guard bytes around the workspace and the output ---------------------------------

GUARD = 4096           # bytes, a multiple of the workspace's 256-byte alignment
PATTERN = 0xA5

# one launch per kernel family that reduces through the workspace
GUARDED = [
    ("w4a16", 1, 1, 5120, 512, 128),     # dot2 with K split across workgroups
    ("w4a16", 2, 5, 5120, 512, 128),     # skinny, split K
    ("w4a16", 3, 128, 2560, 272, 128),   # wide, shared tiles
    ("w4a16", 3, 128, 2560, 272, 32),    # wide, shared tiles, scales in the dequantization
    ("mxfp8", 1, 1, 5120, 512, 32),
    ("mxfp8", 2, 5, 5120, 512, 32),
    ("mxfp8", 3, 128, 2560, 272, 32),
    ("w8a16", 0, 3, 5120, 512, 128),
]


@pytest.mark.parametrize("op,kernel,M,K,N,G", GUARDED, ids=["-".join(map(str, c)) for c in GUARDED])
def test_workspace_and_output_guards(op, kernel, M, K, N, G):
    """The kernels write only inside [workspace, workspace + bytes) and inside
    the output: guard bytes before and after both are untouched after three
    launches, the counters are back at zero and the result passes the gate."""
    import spec_verify_amd as svq
    _say("guards", op, kernel, "M K N G", M, K, N, G)
    if op == "w4a16":
        p = W4(5700 + M + G, M, K, N, G)
        nbytes = p.ws_bytes(kernel)
        run = lambda out, ws: p.run(kernel, out=out, workspace=ws)
        ref = p.ref
    elif op == "mxfp8":
        p = MX(5800 + M, M, K, N)
        nbytes = p.ws_bytes(kernel)
        run = lambda out, ws: p.run(kernel, out=out, workspace=ws)
        ref = p.ref
    else:
        inp = synth.gen_w8a16(5900 + M, M, K, N, G)
        x, w, s = dev(inp.x), dev(inp.w), dev(inp.scales)
        nbytes = svq.w8a16_workspace_bytes(M, N, K)
        run = lambda out, ws: svq.w8a16_gemm(x, w, s, G, out=out, workspace=ws)
        ref = lambda: oracle.w8a16(inp.x, inp.w, inp.scales, G)
    assert nbytes > COUNTER_BYTES                # this launch splits work across workgroups
    wbuf = torch.full((nbytes + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
    wbuf[GUARD:GUARD + nbytes].zero_()
    ws = wbuf[GUARD:GUARD + nbytes]
    og = GUARD // 2                               # output guard, in bf16 elements
    obuf = torch.full((M * N + 2 * og,), 0x7A5A, dtype=torch.int16, device="cuda")
    out = obuf[og:og + M * N].view(M, N).view(torch.bfloat16)
    outs = []
    for _ in range(3):
        run(out, ws)
        outs.append(out.clone())
    torch.cuda.synchronize()
    assert int((wbuf[:GUARD] != PATTERN).sum()) == 0
    assert int((wbuf[GUARD + nbytes:] != PATTERN).sum()) == 0
    assert int((obuf[:og] != 0x7A5A).sum()) == 0 and int((obuf[og + M * N:] != 0x7A5A).sum()) == 0
    assert int(ws[:COUNTER_BYTES].count_nonzero()) == 0
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert_gate(host_bits(out), *ref(), f"guards {op} kernel {kernel}")


# ---- the measurement entry points ----------------------------------------------------

def test_launch_geometry_reports_the_launched_shape():
    import spec_verify_amd as svq
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for op, M, N, K, G in ((1, 1, 6144, 5120, 128), (1, 5, 17408, 5120, 128), (1, 128, 5120, 17408, 128),
                           (2, 1, 5120, 5120, 32), (2, 128, 5120, 5120, 32), (3, 1, 248320, 5120, 128)):
        grid, threads, lds = svq.launch_geometry(op, M, N, K, G)
        _say("geometry", op, M, N, K, G, "->", grid, threads, lds)
        assert 1 <= grid <= 1 << 24 and threads % 64 == 0 and 64 <= threads <= 1024 and lds <= 160 * 1024
        if M == 1 and op == 1:
            assert grid == N // 16                # one workgroup per 16-column block
    # the shape of the workload is that of a real call: a real call still works after the query
    p = W4(6000, 5, 1280, 384, 128)
    out = p.run()
    torch.cuda.synchronize()
    assert_gate(host_bits(out), *p.ref(), "after geometry query")
    assert cus > 0


@pytest.mark.parametrize("grid,threads", [(1, 64), (7, 256), (256, 1024), (1000, 512)])
def test_stream_probe_reads_every_unit(grid, threads):
    """A buffer of zeros with one 32-bit word set to the probe's magic value: the
    lane that reads that 16-byte unit XORs exactly the magic and writes it to the
    sink of its workgroup, so the sink shows which workgroup read the unit."""
    import spec_verify_amd as svq
    nbytes = 1 << 20
    n16 = nbytes // 16
    for unit in (0, 1, n16 // 3, n16 - 1):
        buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        buf[unit * 4 + 2] = 0x5EED5EED
        sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
        svq.stream_probe(buf, nbytes, grid, threads, sink)
        torch.cuda.synchronize()
        owner = next(b for b in range(grid) if b * n16 // grid <= unit < (b + 1) * n16 // grid)
        got = sink.cpu().numpy()
        assert got[owner] == 0x5EED5EED, (unit, owner)
        assert np.count_nonzero(got) == 1


def test_mfma_probe_runs_and_leaves_the_sink():
    """The matrix-core probe runs at several shapes with both operand sets. The
    constant set's sums are positive, and the random set's totals (a fixed
    function of the shape) are not exactly -1, so the store they guard never
    happens and the sink keeps its contents."""
    import spec_verify_amd as svq
    for random_operands in (False, True):
        for grid, threads, per_wave in ((1, 64, 8), (204, 512, 856), (256, 1024, 64)):
            sink = torch.full((grid,), 7.0, dtype=torch.float32, device="cuda")
            svq.mfma_probe(grid, threads, per_wave, sink, random_operands=random_operands)
            torch.cuda.synchronize()
            assert bool((sink == 7.0).all()), (grid, threads, per_wave, random_operands)
