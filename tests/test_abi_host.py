"""The C ABI without a GPU: the library loads, exports every symbol declared in
include/svq.h, and rejects every invalid argument on the host before anything
reaches the HIP runtime (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import spec_verify_amd as svq
    if not os.path.exists(svq.library_path):
        from spec_verify_amd import build
        build.build()
    return svq.lib()


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "svq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(svq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    import spec_verify_amd as svq
    declared = _declared_symbols()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(svq.EXPORTED_SYMBOLS) == declared
    assert L.svq_abi_version() == 1


def test_status_strings(L):
    for code in range(0, 11):
        assert L.svq_status_string(code)
    assert L.svq_status_string(999) == b"unknown status"


FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation first
FAKE2 = 1 << 30
FAKE3 = 1 << 34
FAKE4 = 1 << 38


def _w4(L, M=1, N=256, K=512, G=128, x=FAKE, w=FAKE2, s=FAKE3, o=FAKE4, kernel=0, ws=None, wsb=0):
    return L.svq_w4a16_gemm_with(kernel, x, w, s, o, M, N, K, G, ws, wsb, None)


def test_w4a16_validation(L):
    assert _w4(L, x=None) == 1
    assert _w4(L, o=None) == 1
    assert _w4(L, M=0) == 2
    assert _w4(L, N=-16) == 2
    assert _w4(L, K=1 << 25) == 2
    assert _w4(L, N=1 << 18, K=1 << 13) == 2     # 2^31 weight elements: past the 32-bit offsets
    assert _w4(L, G=16) == 3
    assert _w4(L, G=256) == 3
    assert _w4(L, N=250) == 4
    assert _w4(L, K=320, G=32) == 4          # K % 128
    assert _w4(L, x=FAKE + 2) == 6            # x needs 16-byte alignment
    assert _w4(L, w=FAKE2 + 8) == 6
    assert _w4(L, s=FAKE3 + 1) == 6
    assert _w4(L, s=FAKE3 + 2) == 6
    assert _w4(L, o=FAKE4 + 2) == 6
    assert _w4(L, o=FAKE + 64) == 7            # out overlaps x
    assert _w4(L, M=9, kernel=1) == 10        # dot2 kernel takes M <= 8
    assert _w4(L, M=17, kernel=2) == 10       # skinny kernel takes M <= 16
    assert _w4(L, kernel=7) == 10


def test_mxfp8_validation(L):
    def mx(M=1, N=256, K=512, G=32, x=FAKE, w=FAKE2, s=FAKE3, o=FAKE4, kernel=0):
        return L.svq_mxfp8_gemm_with(kernel, x, w, s, o, M, N, K, G, None, 0, None)
    assert mx(w=None) == 1
    assert mx(K=0) == 2
    assert mx(G=128) == 3
    assert mx(N=96) == 5                      # the N >= 128 constraint, as an error code
    assert mx(K=520) == 5                     # K % 32
    assert mx(K=160) == 4                     # K % 128 (this library's tile height)
    assert mx(N=136) == 4
    assert mx(x=FAKE + 8) == 6
    assert mx(s=FAKE3 + 2) == 6                # scales are read as aligned 32-bit words
    assert mx(o=FAKE2 + 4) == 7
    assert mx(M=9, kernel=1) == 10


def test_repack_validation(L):
    assert L.svq_q4_repack(None, FAKE2, 256, 512, None) == 1
    assert L.svq_q4_repack(FAKE, FAKE2, 0, 512, None) == 2
    assert L.svq_q4_repack(FAKE, FAKE2, 24, 512, None) == 4
    assert L.svq_q4_repack(FAKE, FAKE2, 256, 192, None) == 4
    assert L.svq_q4_repack(FAKE + 4, FAKE2, 256, 512, None) == 6
    assert L.svq_q4_repack(FAKE, FAKE + 4096, 256, 512, None) == 7
    assert L.svq_q4_repacked_bytes(5120, 17408) == 5120 * 17408 // 2
    assert L.svq_q4_repacked_bytes(0, 5) == 0
    assert L.svq_mxfp8_repack(None, FAKE2, 256, 512, None) == 1
    assert L.svq_mxfp8_repack(FAKE, FAKE2, 0, 512, None) == 2
    assert L.svq_mxfp8_repack(FAKE, FAKE2, 24, 512, None) == 4
    assert L.svq_mxfp8_repack(FAKE, FAKE2, 256, 192, None) == 4
    assert L.svq_mxfp8_repack(FAKE + 4, FAKE2, 256, 512, None) == 6
    assert L.svq_mxfp8_repack(FAKE, FAKE + 4096, 256, 512, None) == 7


def test_kernel_selection_names(L):
    name = lambda k, M: L.svq_w4a16_kernel_name(k, M, 5120, 5120, 128)
    assert name(0, 1) == b"w4a16_dot2_kernel"
    assert name(0, 5) == b"w4a16_skinny_kernel"
    assert name(0, 128) == b"w4a16_wide_kernel"
    assert name(1, 9) is None
    assert L.svq_w4a16_kernel_name(0, 1, 5120, 5121, 128) is None
    assert L.svq_mxfp8_kernel_name(0, 1, 5120, 5120) == b"mxfp8_dot2_kernel"
    assert L.svq_mxfp8_kernel_name(0, 5, 5120, 5120) == b"mxfp8_skinny_kernel"
    assert L.svq_mxfp8_kernel_name(0, 128, 5120, 5120) == b"mxfp8_wide_kernel"
    assert L.svq_mxfp8_kernel_name(0, 1, 96, 5120) is None


def test_workspace_query_rejects_bad_shapes(L):
    bad = ctypes.c_size_t(-1).value
    assert L.svq_w4a16_workspace_bytes(0, 1, 5120, 5121, 128) == bad
    assert L.svq_w4a16_workspace_bytes(1, 9, 5120, 5120, 128) == bad
    # enough 16-column blocks to fill the chip: no split of K, no workspace
    assert L.svq_w4a16_workspace_bytes(2, 5, 17408, 5120, 128) == 0
    assert L.svq_w4a16_workspace_bytes(0, 1, 1024, 5120, 128) == 0
    # few column blocks: K is split and the split partials need a workspace
    assert 0 < L.svq_w4a16_workspace_bytes(0, 1, 256, 17408, 128) < (1 << 22)
    assert 0 < L.svq_mxfp8_workspace_bytes(0, 3, 256, 4096) < (1 << 22)
    assert L.svq_mxfp8_workspace_bytes(0, 1, 96, 5120) == bad


def test_w8a16_validation_and_names(L):
    def w8(M=1, N=256, K=512, G=128, x=FAKE, w=FAKE2, s=FAKE3, o=FAKE4):
        return L.svq_w8a16_gemm(x, w, s, o, M, N, K, G, None, 0, None)
    assert w8(w=None) == 1
    assert w8(M=0) == 2
    assert w8(G=96) == 3
    assert w8(N=24) == 4
    assert w8(K=192, G=64) == 4               # K % 128
    assert w8(M=17) == 10                     # one MFMA tile of rows: M <= 16
    assert w8(w=FAKE2 + 8) == 6
    assert w8(s=FAKE3 + 2) == 6
    assert w8(o=FAKE2 + 64) == 7               # out overlaps w
    assert L.svq_w8a16_kernel_name(1, 248320, 5120, 128) == b"w8a16_skinny_kernel"
    assert L.svq_w8a16_kernel_name(17, 256, 512, 128) is None
    bad = ctypes.c_size_t(-1).value
    assert L.svq_w8a16_workspace_bytes(17, 256, 512, 128) == bad
    assert L.svq_w8a16_workspace_bytes(1, 248320, 5120, 128) == 0


def test_rtn_quantize_validation(L):
    def q(w=FAKE, bits=8, G=128, c=FAKE2, s=FAKE3, N=256, K=512):
        return L.svq_rtn_quantize(w, bits, G, c, s, N, K, None)
    assert q(w=None) == 1
    assert q(s=None) == 1
    assert q(N=0) == 2
    assert q(bits=2) == 10
    assert q(G=16) == 3
    assert q(K=96, G=64) == 4
    assert q(w=FAKE + 8) == 6
    assert q(c=FAKE2 + 4) == 6                 # int8 codes are written 16 bytes at a time
    assert q(bits=4, c=FAKE2 + 4, N=0) == 2    # dimensions are checked first
    assert q(s=FAKE3 + 1) == 6
    assert q(c=FAKE + 1024) == 7               # codes overlap w
    assert q(s=FAKE2 + 4096) == 7              # scales overlap codes


def test_fuse_projections_validation(L):
    P = ctypes.c_void_p

    def f(bits=4, ws=(FAKE, FAKE + 65536), ss=(FAKE2, FAKE2 + 65536), widths=(256, 256), parts=None,
          K=512, G=128, wf=FAKE3, sf=FAKE4):
        n = (len(widths) if widths is not None else 2) if parts is None else parts
        wa = (P * max(len(ws), 1))(*ws) if ws is not None else None
        sa = (P * max(len(ss), 1))(*ss) if ss is not None else None
        na = (ctypes.c_int64 * max(len(widths), 1))(*widths) if widths is not None else None
        return L.svq_fuse_projections(bits, wa, sa, na, n, K, G, wf, sf, None)

    assert f(ws=None) == 1
    assert f(widths=None) == 1
    assert f(wf=None) == 1
    assert f(ws=(FAKE, None)) == 1
    assert f(bits=2) == 10
    assert f(parts=0) == 2
    assert f(parts=17, ws=(FAKE,) * 17, ss=(FAKE2,) * 17, widths=(16,) * 17) == 2
    assert f(widths=(256, 0)) == 2
    assert f(K=0) == 2
    assert f(widths=(1 << 24, 16)) == 2            # the fused width is out of range
    assert f(G=16) == 3
    assert f(K=96, G=32) == 4                       # K % 128
    assert f(widths=(256, 24)) == 4                 # a width that is not a multiple of 16
    assert f(ws=(FAKE + 2, FAKE + 65536)) == 6      # GPTQ words are read as 32-bit values
    assert f(bits=8, ws=(FAKE + 4, FAKE + 65536)) == 6   # int8 codes are moved 16 bytes at a time
    assert f(wf=FAKE3 + 4) == 6
    assert f(ss=(FAKE2 + 1, FAKE2 + 65536)) == 6
    assert f(wf=FAKE + 4096) == 7                   # output overlaps a part's weights
    assert f(sf=FAKE2 + 65536 + 64) == 7            # scales output overlaps a part's scales
    assert f(sf=FAKE3 + 1024) == 7                  # the two outputs overlap


def test_ct_to_gptq_validation(L):
    def c(wp=FAKE, ws=FAKE2, qw=FAKE3, s=FAKE4, N=100, K=512, G=128):
        return L.svq_ct_to_gptq(wp, ws, qw, s, N, K, G, None)
    assert c(wp=None) == 1
    assert c(s=None) == 1
    assert c(N=0) == 2
    assert c(K=1 << 25) == 2
    assert c(G=8) == 3
    assert c(K=96, G=64) == 4
    assert c(wp=FAKE + 2) == 6
    assert c(s=FAKE4 + 1) == 6
    assert c(qw=FAKE + 64) == 7
    assert c(s=FAKE3 + 64) == 7


def test_mxfp8_quantize_validation(L):
    def q(w=FAKE, opt=1, c=FAKE2, s=FAKE3, N=256, K=512):
        return L.svq_mxfp8_quantize(w, opt, c, s, N, K, None)
    assert q(w=None) == 1
    assert q(c=None) == 1
    assert q(N=0) == 2
    assert q(K=1 << 25) == 2
    assert q(opt=2) == 10
    assert q(K=48) == 4
    assert q(w=FAKE + 8) == 6
    assert q(c=FAKE2 + 8) == 6
    assert q(c=FAKE + 1024) == 7               # codes overlap w
    assert q(s=FAKE2 + 4096) == 7              # scales overlap codes


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import spec_verify_amd as svq
    monkeypatch.setattr(svq, "_lib", None)
    monkeypatch.setattr(svq, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libsvq.so not found"):
        svq.lib()


def test_format_generic_queries_match_the_per_format_ones(L):
    bad = ctypes.c_size_t(-1).value
    for M in (1, 3, 5, 16, 17, 128):
        for (N, K) in ((5120, 5120), (17408, 5120), (5120, 17408), (256, 1280)):
            assert L.svq_kernel_name(1, M, N, K, 128) == L.svq_w4a16_kernel_name(0, M, N, K, 128)
            assert L.svq_workspace_bytes(1, M, N, K, 64) == L.svq_w4a16_workspace_bytes(0, M, N, K, 64)
            assert L.svq_kernel_name(2, M, N, K, 32) == L.svq_mxfp8_kernel_name(0, M, N, K)
            assert L.svq_workspace_bytes(2, M, N, K, 32) == L.svq_mxfp8_workspace_bytes(0, M, N, K)
            if M <= 16:
                assert L.svq_kernel_name(3, M, N, K, 128) == L.svq_w8a16_kernel_name(M, N, K, 128)
                assert L.svq_workspace_bytes(3, M, N, K, 128) == L.svq_w8a16_workspace_bytes(M, N, K, 128)
    assert L.svq_kernel_name(2, 1, 5120, 5120, 128) is None      # MXFP8 groups are 32
    assert L.svq_workspace_bytes(2, 1, 5120, 5120, 128) == bad
    assert L.svq_kernel_name(0, 1, 5120, 5120, 128) is None      # unknown op
    assert L.svq_workspace_bytes(4, 1, 5120, 5120, 128) == bad
    assert L.svq_kernel_name(3, 17, 5120, 5120, 128) is None     # W8A16 takes M <= 16


def test_launch_geometry_and_stream_probe_validation(L):
    g, t, l = ctypes.c_uint64(), ctypes.c_uint32(), ctypes.c_size_t()
    ref = (ctypes.byref(g), ctypes.byref(t), ctypes.byref(l))
    assert L.svq_launch_geometry(1, 0, 1, 5120, 5121, 128, *ref) == 4     # N % 16
    assert L.svq_launch_geometry(1, 0, 0, 5120, 5120, 128, *ref) == 2
    assert L.svq_launch_geometry(2, 0, 1, 96, 5120, 32, *ref) == 5        # MXFP8 N >= 128
    assert L.svq_launch_geometry(1, 1, 9, 5120, 5120, 128, *ref) == 10    # dot2 takes M <= 8
    assert L.svq_launch_geometry(9, 0, 1, 5120, 5120, 128, *ref) == 10    # unknown op
    assert L.svq_launch_geometry(1, 0, 1, 5120, 5120, 128, None, ref[1], ref[2]) == 1
    assert L.svq_stream_probe(None, 1 << 20, 256, 256, FAKE2, None) == 1
    assert L.svq_stream_probe(FAKE, 1 << 20, 256, 256, None, None) == 1
    assert L.svq_stream_probe(FAKE, 0, 256, 256, FAKE2, None) == 2
    assert L.svq_stream_probe(FAKE, 1000, 256, 256, FAKE2, None) == 2     # not a multiple of 16
    assert L.svq_stream_probe(FAKE, 1 << 20, 0, 256, FAKE2, None) == 2
    assert L.svq_stream_probe(FAKE, 1 << 20, 256, 96, FAKE2, None) == 2   # threads % 64
    assert L.svq_stream_probe(FAKE, 1 << 20, 256, 2048, FAKE2, None) == 2
    assert L.svq_stream_probe(FAKE + 8, 1 << 20, 256, 256, FAKE2, None) == 6
    assert L.svq_stream_probe(FAKE, 1 << 20, 256, 256, FAKE + 64, None) == 7   # sink inside src
    assert L.svq_mfma_probe(256, 512, 64, 0, None, None) == 1
    assert L.svq_mfma_probe(0, 512, 64, 0, FAKE2, None) == 2
    assert L.svq_mfma_probe(256, 96, 64, 0, FAKE2, None) == 2            # threads % 64
    assert L.svq_mfma_probe(256, 2048, 64, 0, FAKE2, None) == 2
    assert L.svq_mfma_probe(256, 512, 0, 0, FAKE2, None) == 2
    assert L.svq_mfma_probe(256, 512, 12, 0, FAKE2, None) == 2           # not a multiple of 8
    assert L.svq_mfma_probe(256, 512, 1 << 25, 0, FAKE2, None) == 2
    assert L.svq_mfma_probe(256, 512, 64, 2, FAKE2, None) == 2           # operands: 0 or 1
    assert L.svq_mfma_probe(256, 512, 64, -1, FAKE2, None) == 2
    assert L.svq_mfma_probe(256, 512, 64, 1, FAKE2 + 2, None) == 6


def test_noalloc_entry_point_validation_without_a_gpu(L):
    # shape errors are those of svq_w4a16_gemm; a workspace beyond the scratch
    # array (2 x 160 tiles over 256 workgroups: 64 MiB of partials) is refused
    assert L.svq_w4a16_gemm_noalloc(FAKE, FAKE2, FAKE3, FAKE4, 1, 5121 - 1 + 8, 5120, 128, None) == 4
    assert L.svq_w4a16_gemm_noalloc(FAKE, FAKE2, FAKE3, FAKE4, 0, 5120, 5120, 128, None) == 2
    assert L.svq_w4a16_gemm_noalloc(FAKE, FAKE2, FAKE3, FAKE4, 1, 5120, 5120, 16, None) == 3
    assert L.svq_w4a16_gemm_noalloc(FAKE, FAKE2, FAKE3, FAKE4, 256, 40960, 5120, 128, None) == 8


def test_narrow_plan_waves_per_unit(L):
    """The narrow-unit GEMV's plan (no device here: 256 CUs assumed): one 4-column
    unit per workgroup at N = 1024, at most four waves per unit, more only where
    eight four-tile loads per wave or four x chunks per thread would not cover K."""
    g, t, l = ctypes.c_uint64(), ctypes.c_uint32(), ctypes.c_size_t()
    geo = lambda M, N, K, G: (L.svq_launch_geometry(1, 1, M, N, K, G, ctypes.byref(g), ctypes.byref(t),
                                                    ctypes.byref(l)), g.value, t.value)
    assert geo(1, 1024, 5120, 128) == (0, 256, 256)      # 10 load groups: 4 waves of 3
    assert geo(1, 1024, 1280, 128) == (0, 256, 192)      # 3 load groups: 3 waves
    assert geo(1, 1024, 17408, 128) == (0, 256, 576)     # 34 groups: x needs 9 waves
    assert geo(1, 4080, 5120, 64) == (0, 255, 1024)      # 4 units per workgroup x 4 waves
    assert L.svq_w4a16_kernel_name(1, 1, 1024, 5120, 128) == b"w4a16_narrow_kernel"
