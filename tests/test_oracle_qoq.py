"""Pins of the oracle's QoQ step (progressive group quantization, W4A8; QoQ/QServe
article, sections "渐进式分组量化" and "W4A8 GEMM的核心设计"): per-channel INT8 in
the protected range [-119, 119], then per-group UINT4 with an integer step and a
zero point whose dequantized values s2 (u - z) stay 8-bit integers, per-token
INT8 activations, one exact integer product over K and a per-channel scale.

Each check compares the oracle with something it does not compute the same way:
exact integer or rational arithmetic, an exhaustive sweep of every group range,
a library int64 matmul of the dequantized 8-bit weights, a float64 matmul, and
closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest

from gen import synth
from tests.test_oracle_pins import f16, small_layer


def round_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_qoq_protected_range_every_group_range(orc):
    """Every range [lo, hi] with -119 <= lo <= 0 <= hi <= 119: the step is
    ceil((hi - lo) / 15) (at least 1), the zero point round(-lo / s2), and every
    value in the range dequantizes to an 8-bit integer (|s2 (u - z)| <= 127, the
    point of the protected range) within s2 / 2 of itself."""
    rng = np.random.default_rng(11)
    worst = 0
    for lo in range(-119, 1):
        for hi in range(0, 120):
            vals = np.concatenate([[lo, hi], rng.integers(lo, hi + 1, 126)]).astype(np.int8)
            s2, z, u = orc.qoq_group(vals)
            assert s2 == max(1, -(-(hi - lo) // 15))
            assert z == round_even(Fraction(-lo, s2)) and 0 <= z <= 15
            deq = s2 * (u.astype(np.int32) - z)
            assert np.all(np.abs(deq) <= 127), (lo, hi)
            assert np.all(np.abs(vals.astype(np.int32) - deq) * 2 <= s2), (lo, hi)
            worst = max(worst, int(np.abs(deq).max()))
    assert worst == 127 or worst <= 127


def test_qoq_group_codes_exhaustive_values(orc):
    """For a sample of ranges, every integer of the range: the code is the nearest
    integer of w / s2 (ties to even) plus z, and the range ends reach 0 and 15 or
    fall within half a step."""
    for lo, hi in ((-119, 119), (-119, 0), (0, 119), (-7, 100), (-60, 3), (0, 0), (-1, 1)):
        vals = np.arange(lo, hi + 1, dtype=np.int8)
        grp = np.resize(vals, 128).astype(np.int8)
        grp[0], grp[1] = lo, hi
        s2, z, u = orc.qoq_group(grp)
        for w, uu in zip(grp, u):
            want = min(15, max(0, round_even(Fraction(int(w), s2)) + z))
            assert uu == want, (lo, hi, w)


def test_qoq_weight_levels(orc):
    """Level 1: s1 = fp16(absmax / 119) per channel, |W - s1 w8| <= s1 / 2 (plus the
    fp32 error of the division) except at the clamped ends; the absmax codes to
    +-119 or stays within half a step. Level 2 dequantizes to 8-bit integers."""
    cfg = synth.CONFIGS["q_proj_7b"]
    W, score = synth.make_w(cfg), synth.make_scores(cfg)
    perm, _ = orc.channel_order(score, 0)
    s1, w8, s2, z, u = orc.qoq_quantize_weights(W, perm)
    a = np.abs(f16(W)).max(1)
    assert np.array_equal(s1, (a / 119).astype(np.float32).astype(np.float16).view(np.uint16))
    s = f16(s1)[:, None]
    wp = f16(W)[:, perm]
    err = np.abs(wp - s * w8)
    assert np.all((err <= s / 2 * (1 + 2.0 ** -20)) | (np.abs(w8) == 119))
    assert np.all(np.abs(w8) <= 119)
    blk = np.arange(cfg.K) // 128
    deq = s2.astype(np.int32)[:, blk] * (u.astype(np.int32) - z.astype(np.int32)[:, blk])
    assert np.all(np.abs(deq) <= 127)
    assert np.all(np.abs(w8 - deq) * 2 <= s2.astype(np.int32)[:, blk])


@pytest.mark.parametrize("name", ["tiny", "q_proj_7b"])
def test_qoq_integer_product(orc, name):
    """P (zero point subtracted after the multiplication, per group) equals an
    int64 matmul of the activation codes and the dequantized 8-bit weights."""
    cfg = synth.CONFIGS[name]
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    rows = (0, min(cfg.M, 16))
    d = orc.qoq_layer(X, W, score, rows)
    blk = np.arange(cfg.K) // 128
    deq = d["s2"].astype(np.int64)[:, blk] * (d["u"].astype(np.int64) - d["z"].astype(np.int64)[:, blk])
    ref = d["qa"][rows[0]:rows[1]].astype(np.int64) @ deq.T
    assert np.array_equal(d["P"].astype(np.int64), ref)


def test_qoq_dequantize_then_matmul(orc):
    """yexact equals a float64 matmul of (s_x q_a) and (s1 s2 (u - z)); Y16 is the fp16
    rounding of y32 = fl(s_x s1) * float(P)."""
    X, W, score, _ = small_layer(24, 512, 40, 29, 0)
    d = orc.qoq_layer(X, W, score)
    blk = np.arange(512) // 128
    A = d["qa"].astype(np.float64) * d["sa"].astype(np.float64)[:, None]
    B = (d["s2"].astype(np.float64)[:, blk] * (d["u"].astype(np.float64) - d["z"].astype(np.float64)[:, blk])
         * f16(d["s1"])[:, None])
    ref, mag = A @ B.T, np.abs(A) @ np.abs(B).T
    assert np.all(np.abs(d["yexact"] - ref) <= 1e-12 * mag + 1e-300)
    t = (d["sa"][:, None] * f16(d["s1"]).astype(np.float32)[None, :]).astype(np.float32)
    assert np.array_equal(d["y32"], (t * d["P"].astype(np.float32)).astype(np.float32))
    assert np.array_equal(d["Y16"], d["y32"].astype(np.float16).view(np.uint16))


def test_qoq_activations_per_token(orc):
    """One scale per token over all K: the absmax element codes to +-127, every code
    is within s/2 of x / s, and an all-zero token gives s = 0, q = 0."""
    cfg = synth.CONFIGS["q_proj_7b"]
    X = synth.make_x(cfg)
    X[3] = 0
    perm, _ = orc.channel_order(synth.make_scores(cfg), 0)
    qa, sa = orc.qoq_quantize_activations(X, perm)
    xp = f16(X)[:, perm]
    assert sa[3] == 0 and np.all(qa[3] == 0)
    live = np.arange(cfg.M) != 3
    assert np.all(np.abs(qa[live]).max(1) == 127)
    err = np.abs(xp - qa * sa.astype(np.float64)[:, None])
    assert np.all(err <= sa.astype(np.float64)[:, None] / 2 + 2.0 ** -22 * np.abs(xp) + 1e-30)


def test_qoq_brute_force_tiny(orc):
    """M = 2, N = 3, K = 256: every step with exact rationals and integers."""
    X, W, score, _ = small_layer(2, 256, 3, 57, 0)
    d = orc.qoq_layer(X, W, score)
    perm = sorted(range(256), key=lambda k: (float(score[k]), k))
    wv, xv = f16(W), f16(X)
    for n in range(3):
        s = float(f16(d["s1"][n]))
        for k in range(256):
            t = Fraction(float(np.float32(wv[n, perm[k]]) / np.float32(s)))
            assert d["w8"][n, k] == max(-119, min(119, round_even(t)))
    for m in range(2):
        for n in range(3):
            p = 0
            for b in range(2):
                s2, z = int(d["s2"][n, b]), int(d["z"][n, b])
                p += sum(int(d["qa"][m, k]) * s2 * (int(d["u"][n, k]) - z) for k in range(128 * b, 128 * b + 128))
            assert d["P"][m, n] == p
            ye = Fraction(float(d["sa"][m])) * Fraction(float(f16(d["s1"][n]))) * p
            assert abs(Fraction(float(d["yexact"][m, n])) - ye) <= abs(ye) * Fraction(1, 2 ** 50)
