"""The seeded input generator: numpy and torch paths agree bit for bit, rows
regenerate independently, and the value recipe has the stated shape."""

import numpy as np
import pytest

import synth


def test_numpy_and_torch_paths_are_bit_identical():
    torch = pytest.importorskip("torch")
    for dt, scale in [("f32", 1.0), ("bf16", 0.02), ("f16", 0.01)]:
        s, _ = synth.quantize_np(synth.normal_np(5, synth.TID_W, 37, 131, scale), dt)
        t = synth.normal_t(5, synth.TID_W, 37, 131, scale, "cpu", dt, row_block=5)
        tv = t.view(torch.int16).numpy().view(np.uint16) if dt == "bf16" else t.numpy()
        assert np.array_equal(s.view(np.uint8), tv.view(np.uint8)), dt
    assert np.array_equal(synth.targets_np(0, 4, 999, 151936),
                          synth.targets_t(0, 4, 999, 151936).numpy())
    # flat indices past 2^32 (the 32768 x 151936 logits reach 4.98e9)
    idx = np.arange(2 ** 32 - 3, 2 ** 32 + 3, dtype=np.uint64)
    assert np.array_equal(synth.bits_np(1, 6, idx).astype(np.int64),
                          synth.bits_t(1, 6, torch.arange(2 ** 32 - 3, 2 ** 32 + 3)).numpy())


def test_rows_regenerate_independently():
    full = synth.normal_np(0, synth.TID_H, 50, 17)
    rows = [3, 49, 0, 22]
    np.testing.assert_array_equal(synth.normal_rows_np(0, synth.TID_H, 17, rows), full[rows])
    w = synth.LinearWorkload("x", 40, 8, 30, "bf16", True, 8, "normal")
    a = synth.make_linear_np(w)
    b = synth.make_linear_np(w, rows=[7, 39])
    np.testing.assert_array_equal(a["h"][[7, 39]], b["h"])
    np.testing.assert_array_equal(a["t"][[7, 39]], b["t"])
    np.testing.assert_array_equal(a["g"][[7, 39]], b["g"])


def test_value_recipe():
    x = synth.normal_np(0, synth.TID_H, 256, 4096)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01
    assert float(np.abs(x).max()) < 4.33
    t = synth.targets_np(0, synth.TID_T, 200000, 1031)
    assert t.min() == 0 and t.max() == 1030
    counts = np.bincount(t, minlength=1031)
    assert counts.min() > 100  # roughly uniform (expected 194 per value)
    bits = synth.f32_to_bf16_bits(np.array([1.0, 1.00390625, 1.01171875, -2.5], np.float32))
    # 1 + 2^-8 is a tie -> rounds to even (1.0); 1 + 3*2^-8 is a tie -> rounds up to 1 + 2^-6
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits), [1.0, 1.0, 1.015625, -2.5])


def test_correct_rounding_reference():
    """round_f64_np is one round-to-nearest-even from float64: it equals numpy's
    own double -> half and double -> float conversions, and for bf16 it picks
    the nearer bf16 neighbour (ties to the even bit pattern)."""
    import numpy as np

    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))
    small = np.abs(x) < 60000
    assert np.array_equal(synth.round_f64_np(x[small], "f16"), x[small].astype(np.float16).astype(np.float64))
    assert np.array_equal(synth.round_f64_np(x, "f32"), x.astype(np.float32).astype(np.float64))
    r = synth.round_f64_np(x, "bf16")
    u = synth.f32_to_bf16_bits(r.astype(np.float32)).astype(np.int32)
    assert np.array_equal(synth.bf16_bits_to_f32(u.astype(np.uint16)).astype(np.float64), r)
    for nb in (u + 1, u - 1):
        v = synth.bf16_bits_to_f32(nb.astype(np.uint16)).astype(np.float64)
        assert np.all(np.abs(x - r) <= np.abs(x - v))
    # exact ties go to the even significand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert synth.round_f64_np(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]), "bf16").tolist() == [1.0, 1 + 2.0 ** -6]
    acc = synth.accuracy(r, x, "bf16")
    assert acc["pct_correctly_rounded"] == 100.0 and acc["max_err_over_max"] <= 2.0 ** -8
