"""GPU: the GEMM entry points under HIP graph capture, for every kernel that
splits work across workgroups (arrival counters in the workspace, which every
call leaves at zero). A graph of three calls is replayed several times with
eager calls and synchronisations in between; every replay must equal the eager
result bit for bit (the reductions run in a fixed order), the counter region
must be zero afterwards, and the result must pass the parity gate against the
oracle. No call records a memset: the kernels clear their own counters.
"""
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


# (label, op, M, K, N, kernel): shapes chosen so that the kernel splits K
# across workgroups (small N for the small-M kernels, several K ranges per tile
# for the wide ones)
CASES = [
    ("w4a16-dot2-split", "w4a16", 1, 5120, 256, 1),
    ("w4a16-skinny-split", "w4a16", 5, 17408, 512, 2),
    # two column blocks per workgroup (x stages would not all fit one per block),
    # a ragged last workgroup, K split three ways: counters cleared per block
    ("w4a16-skinny-multiblock-split", "w4a16", 5, 17408, 5136, 2),
    ("w4a16-wide-streamk", "w4a16", 128, 2048, 1024, 3),
    ("mxfp8-dot2-split", "mxfp8", 2, 4096, 256, 1),
    ("mxfp8-wide-streamk", "mxfp8", 100, 2048, 512, 3),
    ("w8a16-split", "w8a16", 3, 4096, 256, 0),
]


def _setup(op, M, K, N, kernel):
    import spec_verify_amd as svq
    if op == "w4a16":
        inp = synth.gen_w4a16(1200 + M, M, K, N)
        x, w, s = dev(inp.x), svq.q4_repack(dev(inp.qweight)), dev(inp.scales)
        nbytes = svq.w4a16_workspace_bytes(M, N, K, 128, kernel)
        call = lambda o, ws: svq.w4a16_gemm(x, w, s, N, 128, out=o, kernel=kernel, workspace=ws)
        ref = lambda: oracle.w4a16(inp.x, inp.qweight, inp.scales)
    elif op == "mxfp8":
        inp = synth.gen_mxfp8(1300 + M, M, K, N)
        x, w, s = dev(inp.x), svq.mxfp8_repack(dev(inp.w)), dev(inp.scales)
        nbytes = svq.mxfp8_workspace_bytes(M, N, K, kernel)
        call = lambda o, ws: svq.mxfp8_gemm(x, w, s, out=o, kernel=kernel, workspace=ws)
        ref = lambda: oracle.mxfp8(inp.x, inp.w, inp.scales)
    else:
        inp = synth.gen_w8a16(1400 + M, M, K, N)
        x, w, s = dev(inp.x), torch.from_numpy(np.ascontiguousarray(inp.w)).cuda(), dev(inp.scales)
        nbytes = svq.w8a16_workspace_bytes(M, N, K, 128)
        call = lambda o, ws: svq.w8a16_gemm(x, w, s, 128, out=o, workspace=ws)
        ref = lambda: oracle.w8a16(inp.x, inp.w, inp.scales)
    return call, ref, nbytes


@pytest.mark.parametrize("label,op,M,K,N,kernel", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(label, op, M, K, N, kernel):
    _say("graph", label)
    call, ref, nbytes = _setup(op, M, K, N, kernel)
    assert nbytes > COUNTER_BYTES, f"{label}: the shape was meant to split work across workgroups"
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    call(out, ws)
    torch.cuda.synchronize()
    eager = host_u16(out).copy()

    # warm-up on a side stream, then capture three calls into one graph
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            call(out, ws)
    torch.cuda.synchronize()

    for rep in range(5):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), eager, err_msg=f"{label} replay {rep}")
        # eager use of the same workspace between replays
        call(out, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_u16(out), eager, err_msg=f"{label} eager after replay {rep}")
    counters = ws[:COUNTER_BYTES].view(torch.int32).cpu().numpy()
    assert not counters.any(), f"{label}: {np.count_nonzero(counters)} counters left set"
    del g

    y64, y32 = ref()
    ok64, e64, rms = oracle.gate(eager, y64)
    ok32, e32, _ = oracle.gate(eager, y32.astype(np.float64))
    assert ok64 and ok32, f"{label}: err64={e64:.4g} err32={e32:.4g} rms={rms:.4g}"
