"""The seeded generators: reproducible, right shapes, distributions and outliers."""
import numpy as np

import synth


def test_bf16_rounding_is_rne():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    bits = synth.bf16_bits_from_f32(vals)
    back = synth.f32_from_bf16_bits(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even wins (1 + 2^-6)
    assert list(back[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_layer_reproducible_and_shaped():
    cfg = synth.CONFIGS["tiny"]
    a = synth.make_layer(cfg)
    b = synth.make_layer(cfg)
    for name in ("w_up", "w_gate", "w_down", "x_cal", "x_dec", "outlier_pos"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert a.w_up.shape == (256, 768) and a.w_down.shape == (768, 256)
    assert a.x_cal.shape == (64, 256) and a.w_up.dtype == np.float32
    c = synth.make_layer(cfg, layer_index=1)
    assert not np.array_equal(a.w_up, c.w_up)


def test_weight_and_token_distributions():
    cfg = synth.LayerConfig("t", 512, 1024, "bf16", 0.02, 3, 30.0, 64, 0.5, 0.7, 1, 9)
    L = synth.make_layer(cfg)
    assert L.w_up.dtype == np.uint16
    w = synth.as_f64(L.w_gate, "bf16")
    assert abs(w.std() - 0.02) < 0.0005 and abs(w.mean()) < 0.0005
    x = synth.as_f64(L.x_cal, "bf16")
    assert len(L.outlier_pos) == 3 and np.all(np.diff(L.outlier_pos) > 0)
    normal = np.setdiff1d(np.arange(cfg.d_model), L.outlier_pos)
    xn = x[:, normal]
    # Laplace(0,1): mean |x| = 1, var = 2
    assert abs(np.abs(xn).mean() - 1.0) < 0.02 and abs(xn.var() - 2.0) < 0.1
    xo = np.abs(x[:, L.outlier_pos])
    assert abs(xo.mean() - 30.0) < 3.0
