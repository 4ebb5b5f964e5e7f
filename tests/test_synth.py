"""The seeded input generator: determinism and the MXFP8 plain-RTN rule."""
import numpy as np
import pytest

import oracle
import synth


def test_generator_is_deterministic_and_seed_sensitive():
    a = synth.gen_w4a16(201, 1, 512, 64)
    b = synth.gen_w4a16(201, 1, 512, 64)
    c = synth.gen_w4a16(202, 1, 512, 64)
    assert a.digest() == b.digest() != c.digest()
    m1 = synth.gen_mxfp8(501, 2, 256, 128)
    m2 = synth.gen_mxfp8(501, 2, 256, 128)
    assert m1.digest() == m2.digest()


def test_value_ranges():
    inp = synth.gen_w4a16(3, 4, 1024, 64, keep_q=True)
    s = inp.scales.view(np.float16).astype(np.float64)
    assert s.min() >= 0.0019 and s.max() <= 0.0201
    assert inp.q.min() == 0 and inp.q.max() == 15
    x = oracle.bf16_bits_to_f64(inp.x)
    assert abs(x.mean()) < 0.1 and 0.9 < x.std() < 1.1


def test_e4m3_encoder_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(2000) * 0.01,
                        np.array([0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10, 0.5])])
    v = np.clip(v, -448, 448).astype(np.float32)
    ours = synth.e4m3_encode_rne(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0 vs +0 on underflow is the only tolerated difference
    diff = ours != ref
    assert np.all((ours[diff] & 0x7F) == 0) and np.all((ref[diff] & 0x7F) == 0)


def test_mxfp8_rtn_block_rule():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((16, 256)).astype(np.float32)
    W[3, 32:64] = 0.0
    codes, sc = synth.mxfp8_quantize_rtn(W)
    table = oracle.e4m3_table()
    assert sc[3, 1] == 127 and np.all(codes[3, 32:64] & 0x7F == 0)
    amax = np.abs(W.reshape(16, 8, 32)).max(axis=2)
    for n in range(16):
        for b in range(8):
            if amax[n, b] == 0:
                continue
            X = int(np.floor(np.log2(amax[n, b]))) - 8
            assert sc[n, b] == X + 127
            deq = table[codes[n, 32 * b:32 * b + 32]] * 2.0 ** X
            # RTN: every element within half an E4M3 step of its block-scaled value
            v = W[n, 32 * b:32 * b + 32].astype(np.float64)
            step = np.where(np.abs(v) / 2.0 ** X < 2 ** -6, 2.0 ** -9,
                            2.0 ** (np.floor(np.log2(np.maximum(np.abs(v) / 2.0 ** X, 2 ** -6))) - 3))
            err = np.abs(deq - v) / 2.0 ** X
            clipped = np.abs(v) / 2.0 ** X > 448
            assert np.all(err[~clipped] <= step[~clipped] / 2 + 1e-12)
            assert np.all(np.abs(deq[clipped]) / 2.0 ** X == 448)


def test_workload_table_shapes():
    for name, w in synth.WORKLOADS.items():
        assert w["K"] % 128 == 0 and w["N"] % 16 == 0, name
