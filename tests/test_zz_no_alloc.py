"""The allocation-free W4A16 entry point (svq_w4a16_gemm_noalloc) through the C
ABI, against the existing entry point (svq_w4a16_gemm with a caller workspace)
and the oracle: two calls in a row on one device, the second with a smaller
input, so the second reuses the scratch array the first left behind. The same
kernels run in the same order, so the bits must be identical; both also pass
the parity gate against the fp64 and fp32-sequential oracle.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    import spec_verify_amd as svq
    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    return svq.lib()


def _say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


SCRATCH_BYTES = (32 << 20) + (256 << 10)   # SVQ_NOALLOC_SCRATCH_BYTES


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _problem(seed, M, K, N, G):
    import spec_verify_amd as svq
    inp = synth.gen_w4a16(seed, M, K, N, G)
    return inp, dev(inp.x), svq.q4_repack(dev(inp.qweight)), dev(inp.scales)


def _existing(L, x, tiled, s, M, N, K, G):
    import spec_verify_amd as svq
    nb = svq.w4a16_workspace_bytes(M, N, K, G)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = L.svq_w4a16_gemm(ptr(x), ptr(tiled), ptr(s), ptr(out), M, N, K, G, ptr(ws) if nb else None,
                          nb, stream())
    assert st == 0
    return out, nb


def _noalloc(L, x, tiled, s, M, N, K, G):
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = L.svq_w4a16_gemm_noalloc(ptr(x), ptr(tiled), ptr(s), ptr(out), M, N, K, G, stream())
    assert st == 0, st
    return out


# Each pair: a first call, then a smaller one. The shapes split work across
# workgroups, so the scratch array carries counters and partials: the wide
# kernel's shared tiles (M = 128), the skinny kernel's split K (M = 5, 32 column
# blocks) and the decode kernel's split K (M = 1, 32 column blocks); the last
# pair's second call needs no scratch at all.
PAIRS = [
    ((128, 2560, 512, 128), (64, 1280, 256, 32)),
    ((128, 5120, 512, 64), (5, 5120, 512, 128)),
    ((5, 5120, 512, 128), (1, 5120, 512, 128)),
    ((17, 2560, 272, 128), (1, 1280, 6144, 128)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a}->{b}" for a, b in PAIRS])
def test_noalloc_matches_the_workspace_entry_point(L, first, second):
    for i, (M, K, N, G) in enumerate((first, second)):
        _say("noalloc call", i, "M K N G", M, K, N, G)
        inp, x, tiled, s = _problem(9000 + 7 * M + K + N + G, M, K, N, G)
        got = _noalloc(L, x, tiled, s, M, N, K, G)
        ref, nb = _existing(L, x, tiled, s, M, N, K, G)
        torch.cuda.synchronize()
        if i == 0:
            assert nb > 0            # the first call of each pair uses the scratch array
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (M, K, N, G)
        y64, y32 = oracle.w4a16(inp.x, inp.qweight, inp.scales, G)
        for y in (y64, y32.astype(np.float64)):
            ok, err, rms = oracle.gate(host_bits(got), y)
            assert ok, f"noalloc M{M} K{K} N{N} G{G}: err={err:.4g} rms={rms:.4g}"


def test_noalloc_rejects_workspace_beyond_the_scratch_and_bad_arguments(L):
    import spec_verify_amd as svq
    # 2 x 160 tiles of 128 x 256 over 256 workgroups: each takes parts of two
    # tiles, 64 MiB of partials, more than the scratch array holds
    M, N, K = 256, 40960, 5120
    assert svq.w4a16_workspace_bytes(M, N, K, 128) > SCRATCH_BYTES
    fake = 1 << 40
    assert L.svq_w4a16_gemm_noalloc(fake, fake * 2, fake * 3, fake * 4, M, N, K, 128, None) == 8
    # argument errors are those of svq_w4a16_gemm, reported before anything runs
    assert L.svq_w4a16_gemm_noalloc(None, fake * 2, fake * 3, fake * 4, 5, 512, 5120, 128, None) == 1
    assert L.svq_w4a16_gemm_noalloc(fake, fake * 2, fake * 3, fake * 4, 5, 500, 5120, 128, None) == 4
    assert L.svq_w4a16_gemm_noalloc(fake + 2, fake * 2, fake * 3, fake * 4, 5, 512, 5120, 128, None) == 6
