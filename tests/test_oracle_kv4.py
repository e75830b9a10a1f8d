"""Pins of the oracle's KV4 decode attention (step 9 of the oracle: QoQ/QServe
article, section "KV4注意力Kernel优化" -- 4-bit keys and values quantized per
head and token with an fp16 scale and zero point; COMET article: the KV cache
compressed to 4 bits).

The codes are checked against exact rational arithmetic and closed forms for
special vectors; the attention against closed forms that a dropped term, a
wrong scale, a wrong sign or a mixed-up index fails: one cached token, equal
keys, a zero query, two tokens (a logistic of the score gap), the
convex-hull bound, and invariance under a permutation of the tokens and of
the heads.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.test_oracle_pins import f16


def nearest(t: Fraction) -> int:
    fl = t.numerator // t.denominator
    return fl + 1 if t - fl > Fraction(1, 2) else fl


def near_half(t: Fraction, tol=Fraction(1, 10**5)) -> bool:
    fl = t.numerator // t.denominator
    return abs((t - fl) - Fraction(1, 2)) <= tol


def h16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def dequant(u, s16, z):
    """s (u - z) per vector, float64, from the stored parts."""
    return f16(s16)[..., None] * (u.astype(np.float64) - z.astype(np.float64)[..., None])


def cache(rng, H, T, d, scale=1.0):
    K = (rng.standard_normal((H, T, d)) * scale).astype(np.float16)
    V = (rng.standard_normal((H, T, d)) * scale).astype(np.float16)
    return K, V


def quant(orc, C):
    H, T, d = C.shape
    u, s, z = orc.kv4_quantize(C.reshape(H * T, d).view(np.uint16))
    return u.reshape(H, T, d), s.reshape(H, T), z.reshape(H, T)


def attend(orc, q, Kq, Vq):
    return orc.kv4_attention(q.view(np.uint16), *Kq, *Vq)


# ---------------------------------------------------------------- codes

def test_kv4_codes_against_rationals(orc):
    """z is the nearest integer of -15 lo / (hi - lo), each code the nearest
    integer of 15 v / (hi - lo) plus z (clamped to [0, 15]), and the fp16 step
    is within half an fp16 ulp (plus the binary32 rounding before it) of
    (hi - lo) / 15."""
    rng = np.random.default_rng(11)
    for trial in range(400):
        d = int(rng.choice([8, 64, 128]))
        v = (rng.standard_normal(d) * 10 ** rng.uniform(-3, 3)).astype(np.float16)
        if trial % 5 == 0:
            v = np.abs(v)                        # all non-negative: lo = 0
        if trial % 7 == 0:
            v = -np.abs(v)                       # all non-positive: hi = 0
        u, s, z = orc.kv4_quantize(v.view(np.uint16)[None, :])
        vals = [Fraction(float(x)) for x in v]
        lo, hi = min(min(vals), Fraction(0)), max(max(vals), Fraction(0))
        if lo == hi:
            assert s[0] == 0 and z[0] == 0 and not u.any()
            continue
        rng_ = hi - lo
        step = float(f16(s)[0])
        assert abs(Fraction(step) - rng_ / 15) <= rng_ / 15 * Fraction(1, 2**11) * (1 + Fraction(1, 2**12)) \
            or s[0] == 1
        t = -lo * 15 / rng_
        if not near_half(t):
            assert int(z[0]) == min(15, max(0, nearest(t)))
        for i, x in enumerate(vals):
            c = x * 15 / rng_
            if near_half(c):
                continue
            want = min(15, max(0, nearest(c) + int(z[0])))
            assert int(u[0, i]) == want, (trial, i, float(x), int(u[0, i]), want)


def test_kv4_special_vectors(orc):
    """Closed forms: an all-positive vector has z = 0 and its maximum codes to 15;
    an all-negative one z = 15 and its minimum codes to 0; zero channels code to
    u = z, so zero is represented exactly; a zero vector gets step 0."""
    pos = np.array([0.5, 1.0, 3.0, 7.5, 0.0, 2.0, 6.0, 1.5], np.float16)
    u, s, z = orc.kv4_quantize(pos.view(np.uint16)[None, :])
    assert z[0] == 0 and u[0, 3] == 15 and u[0, 4] == 0
    assert float(f16(s)[0]) == 0.5                     # 7.5 / 15, exact in fp16
    assert list(u[0]) == [1, 2, 6, 15, 0, 4, 12, 3]
    neg = -pos
    u, s, z = orc.kv4_quantize(neg.view(np.uint16)[None, :])
    assert z[0] == 15 and u[0, 3] == 0 and u[0, 4] == 15
    mixed = np.array([-3.0, 0.0, 4.5, 0.0, -1.5, 1.5, 0.0, 0.75], np.float16)
    u, s, z = orc.kv4_quantize(mixed.view(np.uint16)[None, :])
    assert float(f16(s)[0]) == 0.5 and z[0] == 6
    assert list(u[0]) == [0, 6, 15, 6, 3, 9, 6, 8]    # 0.75 / 0.5 = 1.5 -> 2 (rint even)
    zero = np.zeros(16, np.float16)
    u, s, z = orc.kv4_quantize(zero.view(np.uint16)[None, :])
    assert s[0] == 0 and z[0] == 0 and not u.any()


def test_kv4_round_trip_bound(orc):
    """Each dequantized channel is within one step (half a step of rounding,
    plus what the clamp at the range ends and the fp16 step add) of the value."""
    rng = np.random.default_rng(5)
    C = (rng.standard_normal((512, 128)) * rng.uniform(0.01, 50, (512, 1))).astype(np.float16)
    u, s, z = orc.kv4_quantize(C.view(np.uint16))
    back = dequant(u, s, z)
    x = C.astype(np.float64)
    rng_ = np.maximum(x.max(1), 0) - np.minimum(x.min(1), 0)
    step = rng_ / 15
    err = np.abs(back - x)
    bound = step[:, None] * (1.0 + 2.0**-9) + 15 * np.abs(f16(s) - step)[:, None]
    assert (err <= bound).all()
    # mean error is about a quarter step for uniform rounding error
    assert 0.15 < float((err / step[:, None]).mean()) < 0.35


# ---------------------------------------------------------------- attention

def test_kv4_attention_one_token(orc):
    """With one cached token the softmax weight is 1: out = dequantized v_0."""
    rng = np.random.default_rng(1)
    K, V = cache(rng, 4, 1, 64)
    q = rng.standard_normal((4, 64)).astype(np.float16)
    Kq, Vq = quant(orc, K), quant(orc, V)
    out = attend(orc, q, Kq, Vq)
    assert np.array_equal(out, dequant(*Vq)[:, 0, :])


def test_kv4_attention_equal_keys_and_zero_query(orc):
    """Equal keys, or a zero query, give equal weights: out = the mean of the
    dequantized values."""
    rng = np.random.default_rng(2)
    H, T, d = 3, 37, 128
    K, V = cache(rng, H, T, d)
    K[:] = K[:, :1, :]
    q = rng.standard_normal((H, d)).astype(np.float16)
    Kq, Vq = quant(orc, K), quant(orc, V)
    want = dequant(*Vq).mean(axis=1)
    np.testing.assert_allclose(attend(orc, q, Kq, Vq), want, rtol=1e-12, atol=1e-12)
    K2, _ = cache(rng, H, T, d)
    out0 = attend(orc, np.zeros((H, d), np.float16), quant(orc, K2), Vq)
    np.testing.assert_allclose(out0, want, rtol=1e-12, atol=1e-12)


def test_kv4_attention_two_tokens_logistic(orc):
    """Two tokens: the first weight is 1 / (1 + exp((a_1 - a_0))) with
    a_t = q . k_t / sqrt(d), the score taken from a one-hot query on a channel
    whose dequantized key values are known exactly."""
    d = 64
    for c, (k0, k1) in enumerate([(4.0, -2.0), (-1.5, 3.0), (7.5, 7.0)]):
        K = np.zeros((1, 2, d), np.float16)
        K[0, 0, :] = np.linspace(-1, 1, d)
        K[0, 1, :] = np.linspace(1, -1, d)
        K[0, 0, c] = k0
        K[0, 1, c] = k1
        V = np.zeros((1, 2, d), np.float16)
        V[0, 0, :] = 1.0
        V[0, 1, :] = -1.0
        V[0, 0, 0] = V[0, 1, 0] = 0.0            # keep zero in range exactly
        q = np.zeros((1, d), np.float16)
        q[0, c] = 2.0
        Kq, Vq = quant(orc, K), quant(orc, V)
        kd = dequant(*Kq)[0, :, c]               # exact dequantized key values
        a0, a1 = 2.0 * kd[0] / np.sqrt(d), 2.0 * kd[1] / np.sqrt(d)
        p0 = 1.0 / (1.0 + np.exp(a1 - a0))
        vd = dequant(*Vq)[0]
        want = p0 * vd[0] + (1 - p0) * vd[1]
        np.testing.assert_allclose(attend(orc, q, Kq, Vq)[0], want, rtol=1e-12, atol=1e-14)


def test_kv4_attention_dominant_key(orc):
    """A key far better aligned with the query than the rest takes all the
    weight: out tends to that token's value."""
    rng = np.random.default_rng(4)
    H, T, d = 2, 50, 128
    K, V = cache(rng, H, T, d, scale=0.05)
    q = np.ones((H, d), np.float16)
    K[0, 17, :] = 8.0
    K[1, 3, :] = 8.0
    Kq, Vq = quant(orc, K), quant(orc, V)
    out = attend(orc, q, Kq, Vq)
    vd = dequant(*Vq)
    np.testing.assert_allclose(out[0], vd[0, 17], atol=1e-12)
    np.testing.assert_allclose(out[1], vd[1, 3], atol=1e-12)


def test_kv4_attention_hull_and_permutations(orc):
    """out lies in the convex hull of the values per channel; permuting the
    cached tokens leaves it unchanged and permuting the heads permutes it."""
    rng = np.random.default_rng(6)
    H, T, d = 5, 200, 128
    K, V = cache(rng, H, T, d, scale=3.0)
    q = (rng.standard_normal((H, d)) * 2).astype(np.float16)
    Kq, Vq = quant(orc, K), quant(orc, V)
    out = attend(orc, q, Kq, Vq)
    vd = dequant(*Vq)
    assert (out >= vd.min(axis=1) - 1e-12).all() and (out <= vd.max(axis=1) + 1e-12).all()
    assert np.abs(out).max() > 0.05                   # not trivially averaged away
    perm = rng.permutation(T)
    Kp = tuple(a[:, perm] for a in Kq)
    Vp = tuple(a[:, perm] for a in Vq)
    np.testing.assert_allclose(attend(orc, q, Kp, Vp), out, rtol=1e-12, atol=1e-13)
    hp = rng.permutation(H)
    out_h = attend(orc, q[hp], tuple(a[hp] for a in Kq), tuple(a[hp] for a in Vq))
    np.testing.assert_allclose(out_h, out[hp], rtol=0, atol=0)


def test_kv4_attention_rejects_empty(orc):
    with pytest.raises(Exception):
        orc.kv4_quantize(np.zeros((0, 8), np.uint16))
