"""The seeded input generator: shapes, determinism, bf16 rounding."""
import numpy as np

from workload import CONFIGS, bf16_bits_to_f32, make_inputs, round_to_bf16, sample_row_blocks


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, 1.0 + 3 * 2 ** -8, -2.5, 0.0,
                     3.14159265, 1e-30, -65504.0], dtype=np.float32)
    r, bits = round_to_bf16(vals)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1; 1 + 3*2^-8 -> 1 + 2^-6
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6, -2.5, 0.0, 3.140625, 1e-30, -65536.0])
    assert np.allclose(r[[0, 1, 2, 3, 4, 5, 6, 8]], expect[[0, 1, 2, 3, 4, 5, 6, 8]], rtol=0, atol=0)
    assert np.array_equal(bf16_bits_to_f32(bits), r)
    # every rounded value is exactly representable: low 16 bits are zero
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_inputs_shapes_and_determinism():
    cfg = CONFIGS["tiny"]
    a = make_inputs(cfg, seed=0)
    b = make_inputs(cfg, seed=0)
    assert a.x.shape == (1, 128, 256) and a.w_in.shape == (3 * 256 + 1024, 256) and a.w_out.shape == (256, 1280)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_in, b.w_in)
    assert a.x.dtype == np.float32 and a.bits is None
    assert np.all(a.gamma == 1) and np.all(a.beta == 0)
    c = make_inputs(cfg, seed=1)
    assert not np.array_equal(a.x, c.x)
    assert abs(a.w_in.std() - 0.02) < 1e-3 and abs(a.x.std() - 1) < 2e-2


def test_bf16_inputs_small_shape():
    cfg = CONFIGS["small"].replace(B=1, S=64, d=128, H=2, hd=64, ffn=256, W=16)
    inp = make_inputs(cfg, seed=0, affine=True)
    for k in ("x", "gamma", "beta", "w_in", "w_out"):
        assert inp.bits[k].dtype == np.uint16
        assert np.array_equal(bf16_bits_to_f32(inp.bits[k]).reshape(getattr(inp, k).shape), getattr(inp, k))
    assert np.abs(inp.gamma - 1).max() > 0


def test_flop_counts_match_tables():
    # algorithmic GFLOP per forward: GEMMs plus attention over in-window pairs
    expect = {"small": 419.8, "shard175b": 933.4, "long": 3427.4, "fullcausal": 3573.5}
    for name, gf in expect.items():
        assert abs(CONFIGS[name].flops() / 1e9 - gf) < 0.1, name
    c = CONFIGS["shard175b"]
    assert c.keys_per_head() == 2048 * 512 - 512 * 511 // 2
    f = CONFIGS["fullcausal"]
    assert f.keys_per_head() == 4096 * 4097 // 2


def test_row_blocks_cover_edges():
    cfg = CONFIGS["long"]
    blocks = sample_row_blocks(cfg)
    assert (0, 0, 32) in blocks and (0, cfg.S - 32, cfg.S) in blocks
    for b, i0, i1 in blocks:
        assert 0 <= i0 < i1 <= cfg.S and 0 <= b < cfg.B
