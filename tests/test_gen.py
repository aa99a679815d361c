"""Input generator: determinism, storage encoders and planted structure."""
import numpy as np
import torch

import gen
from tests import brute


def test_bf16_encoder_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.bf16_bits(x), ref)


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 60,
                        rng.standard_normal(20000).astype(np.float32) * 0.01,
                        np.array([448.0, -448.0, 0.0, 2 ** -6, 2 ** -9, 2 ** -10, 3 * 2 ** -10,
                                  1.0625, 1.1875], np.float32)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = gen.e4m3fn_bits(x)
    # -0.0 vs 0.0 for values that round to zero may differ only in the sign bit
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert same.all()


def test_e4m3_encoder_saturates():
    got = gen.e4m3fn_bits(np.array([500.0, -1e6, 460.0], np.float32))
    assert got.tolist() == [0x7E, 0xFE, 0x7E]


def test_deterministic_per_seed():
    a = gen.make_config(1, seq=512)
    b = gen.make_config(1, seq=512)
    c = gen.make_config(1, seed=99, seq=512)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert not np.array_equal(a.q, c.q)


def test_config_shapes_and_dtypes():
    for i, dt, store in [(0, "f32", np.float32), (1, "bf16", np.uint16), (4, "fp8", np.uint8)]:
        c = gen.make_config(i, seq=256)
        cfg = gen.CONFIGS[i]
        assert c.dtype == dt and c.q.dtype == store
        assert c.q.shape == (cfg["hq"], 256, cfg["d"]) and c.k.shape == (cfg["hkv"], 256, cfg["d"])
    c = gen.make_config(4, seq=256)
    assert c.q_scale.shape == (28,) and c.k_scale.shape == (4,) and c.v_scale.shape == (4,)
    q = brute.decode(c.q, "fp8")
    assert np.isclose(np.abs(q).max(axis=(1, 2)), 448).all()


def test_planted_vertical_keys_stand_out():
    c = gen.make_case(2, 1, 2048, 64, 64, "f32", 5, n_vert=8)
    rng = np.random.Generator(np.random.PCG64(5))
    u = rng.standard_normal(64)
    u /= np.linalg.norm(u)
    pos = np.sort(rng.choice(2048, size=8, replace=False))
    proj = c.k[0] @ u
    assert np.all(proj[pos] > 2.0)
    assert np.abs(np.delete(proj, pos)).mean() < 1.0
    # every query carries +u
    assert abs((c.q[0] @ u).mean() - 1.0) < 0.1


def test_rope_preserves_pair_norms():
    a = gen.make_case(1, 1, 64, 8, 32, "f32", 3, rope=False)
    b = gen.make_case(1, 1, 64, 8, 32, "f32", 3, rope=True)
    na = a.q[0, :, :4] ** 2 + a.q[0, :, 4:] ** 2
    nb = b.q[0, :, :4] ** 2 + b.q[0, :, 4:] ** 2
    np.testing.assert_allclose(na, nb, rtol=1e-5)
    np.testing.assert_array_equal(a.q[0, 0], b.q[0, 0])  # position 0 is not rotated


def test_random_block_mask_structure():
    m = gen.random_block_mask(3, 16, 0.1, 0)
    assert m.shape == (3, 16, 16)
    assert np.all(np.triu(m, 1) == 0)
    assert np.all(m[:, :, 0] == 1) and np.all(m[:, np.arange(16), np.arange(16)] == 1)
