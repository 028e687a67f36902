"""Host check of the decomposition the MFMA router relies on for a float32 W_g:
w = hi + mid + lo with hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid)
(round to nearest even at every step). The three bf16 planes hold w to within
2^-27 |w|, and every product with a bf16 x is exact in float32 (8 + 8
significand bits), so the sum of the three plane products is a float32
dot product up to accumulation order. Pure numpy; no GPU."""
import numpy as np


def bf16_round(a):
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def planes(w):
    w = np.asarray(w, np.float32)
    hi = bf16_round(w)
    r1 = (w - hi).astype(np.float32)
    mid = bf16_round(r1)
    lo = bf16_round((r1 - mid).astype(np.float32))
    return hi, mid, lo


def test_bf16_round_matches_known_values():
    assert bf16_round(np.float32(1.0)) == 1.0
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert bf16_round(np.float32(1.0 + 2.0 ** -8)) == 1.0
    assert bf16_round(np.float32(1.0 + 3 * 2.0 ** -8)) == np.float32(1.0 + 2.0 ** -6)
    assert bf16_round(np.float32(-2.5)) == -2.5


def test_three_planes_hold_float32_weights():
    rng = np.random.default_rng(0)
    for scale in (1e-3, 0.02, 1.0, 300.0):
        w = (rng.standard_normal(200000) * scale).astype(np.float32)
        hi, mid, lo = planes(w)
        rec = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
        err = np.abs(rec - w.astype(np.float64))
        assert np.all(err <= 2.0 ** -27 * np.abs(w.astype(np.float64)) + 1e-45)
        # most weights are reproduced exactly
        assert np.mean(err == 0) > 0.9


def test_plane_products_are_exact_in_float32():
    rng = np.random.default_rng(1)
    x = bf16_round(rng.standard_normal(100000).astype(np.float32))
    w = rng.standard_normal(100000).astype(np.float32) * 0.05
    for p in planes(w):
        prod32 = (x * p).astype(np.float32)
        assert np.array_equal(prod32.astype(np.float64), x.astype(np.float64) * p.astype(np.float64))


def test_logits_from_planes_match_a_float64_dot_product():
    # the float32 router's logits to within float32 accumulation error
    rng = np.random.default_rng(2)
    T, d, E = 64, 1024, 8
    x = bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    w = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    hi, mid, lo = planes(w)
    acc = np.zeros((T, E), np.float32)
    for p in (hi, mid, lo):
        acc = (acc + (x @ p.T).astype(np.float32)).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    scale = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert np.all(np.abs(acc - ref) <= 4 * d * 2.0 ** -24 * scale + 1e-30)
