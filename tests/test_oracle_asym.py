"""Pins of the oracle's asymmetric 4-bit activation variant (step 3b of the
oracle: QUIK blog, section "反量化背后的数学" -- activations with a scale and
a zero point, weights with a scale only, the zero-point term carried by the
offline weight sum).

As for the symmetric path, every check compares the oracle with something it
does not compute the same way: exact rational arithmetic, closed forms for
special blocks, a brute-force enumeration, a float64 matmul of the dequantized
operands, and the identity between the zero-point form of the partials and
the signed-code form.
"""
from fractions import Fraction

import numpy as np
import pytest

from gen import synth
from tests.test_oracle_pins import _correctly_rounded_f32, f16, small_layer


def nearest(t: Fraction) -> int:
    """Nearest integer of t (only called away from half-way points)."""
    fl = t.numerator // t.denominator
    return fl + 1 if t - fl > Fraction(1, 2) else fl


def near_half(t: Fraction, tol=Fraction(1, 10**5)) -> bool:
    fl = t.numerator // t.denominator
    return abs((t - fl) - Fraction(1, 2)) <= tol


def test_asym_params_against_rationals(orc):
    """inv = 15/d and s = d/15 correctly rounded (d = hi - lo, exact here), z the
    nearest integer of -15 lo / d, and the range ends code to 0 and 15."""
    rng = np.random.default_rng(3)
    mags = f16(np.arange(1, 0x7C00, 97, dtype=np.uint16))
    for _ in range(3000):
        lo = -float(rng.choice(mags)) if rng.random() < 0.9 else 0.0
        hi = float(rng.choice(mags)) if rng.random() < 0.9 or lo == 0.0 else 0.0
        if abs(np.log2(max(hi, 1e-30) / max(-lo, 1e-30))) > 12:
            continue                       # keep hi - lo exact in binary32
        inv, s, z = orc.act_asym_params(lo, hi)
        d = Fraction(hi) - Fraction(lo)
        assert float(np.float32(hi) - np.float32(lo)) == float(d)
        assert _correctly_rounded_f32(Fraction(15) / d, inv)
        assert _correctly_rounded_f32(d / 15, s)
        assert 0 <= z <= 15
        t = -Fraction(lo) * 15 / d
        if not near_half(t):
            assert z == nearest(t)
        u_lo = orc.act_asym_code(lo, inv, z)
        u_hi = orc.act_asym_code(hi, inv, z)
        if not near_half(t):
            assert u_lo == 0 and u_hi == 15, (lo, hi, z, u_lo, u_hi)


def test_asym_special_blocks(orc):
    """Closed forms: an all-positive block has z = 0 and its maximum codes to 15;
    an all-negative one z = 15 and its minimum codes to 0; zero codes to u = z
    (zero is represented exactly); an all-zero block gets step 0, zero point 0."""
    K = 512
    X = np.zeros((4, K), np.float16)
    rng = np.random.default_rng(5)
    X[0] = np.abs(rng.standard_normal(K)).astype(np.float16) + np.float16(0.01)   # all positive
    X[1] = -np.abs(rng.standard_normal(K)).astype(np.float16) - np.float16(0.01)  # all negative
    X[2] = rng.standard_normal(K).astype(np.float16)
    X[2, ::7] = 0                                                                  # planted zeros
    X[3, 128:256] = rng.standard_normal(128).astype(np.float16)                   # other blocks zero
    perm = np.arange(K, dtype=np.int32)
    flags = np.zeros(K // 128, np.uint8)
    qa, u4, sa, za = orc.quantize_activations_asym(X.view(np.uint16), perm, flags)
    x = X.astype(np.float64)
    assert np.all(za[0] == 0)
    assert np.all(za[1] == 15)
    for b in range(4):
        blk = slice(128 * b, 128 * b + 128)
        assert u4[0, blk][np.argmax(x[0, blk])] == 15
        assert u4[1, blk][np.argmin(x[1, blk])] == 0
        assert np.float32(sa[0, b]) == np.float32(np.float32(x[0, blk].max()) / np.float32(15))
    z2 = za[2][np.arange(K) // 128]
    assert np.all(u4[2][x[2] == 0] == z2[x[2] == 0])
    assert np.all(qa[2][x[2] == 0] == 0)
    for b in (0, 2, 3):
        blk = slice(128 * b, 128 * b + 128)
        assert sa[3, b] == 0 and za[3, b] == 0 and np.all(u4[3, blk] == 0) and np.all(qa[3, blk] == 0)
    assert sa[3, 1] > 0
    assert np.array_equal(qa.astype(np.int32), u4.astype(np.int32) - za[:, np.arange(K) // 128])


@pytest.mark.parametrize("name", ["q_proj_7b", "down_7b"])
def test_asym_round_trip_and_step(orc, name):
    """x ~ s (u - z) within s/2 (plus the fp32 error of the product) except where the
    code is clamped at a range end (then within s); the step is at most 2/15 of the
    block's absmax, below the symmetric 4-bit step absmax/7; 8-bit blocks equal the
    symmetric path's."""
    cfg = synth.CONFIGS[name]
    X = synth.make_x(cfg)
    score = synth.make_scores(cfg)
    perm, flags = orc.channel_order(score, cfg.nb8)
    qa, u4, sa, za = orc.quantize_activations_asym(X, perm, flags)
    qs, ss = orc.quantize_activations(X, perm, flags)
    blk = np.arange(cfg.K) // 128
    xp = f16(X)[:, perm]
    s = sa.astype(np.float64)[:, blk]
    err = np.abs(xp - qa * s)
    is4 = flags[blk] == 0
    clamped = (u4 == 0) | (u4 == 15)
    ok = err <= s / 2 + 2.0 ** -22 * np.abs(xp) + 1e-30
    assert np.all(ok | (is4[None, :] & clamped & (err <= s * (1 + 2.0 ** -20))))
    assert np.all(u4 <= 15) and np.all(za <= 15)
    a = np.abs(xp).reshape(cfg.M, cfg.nb, 128).max(-1)
    f4 = flags == 0
    assert np.all(sa[:, f4] <= (2.0 / 15) * a[:, f4] * (1 + 2.0 ** -22))
    assert np.all(sa[:, f4] < ss[:, f4] + (ss[:, f4] == 0))
    # 8-bit blocks: identical to the symmetric quantizer, zero point 0
    f8 = flags == 1
    assert np.array_equal(sa[:, f8], ss[:, f8]) and np.all(za[:, f8] == 0)
    assert np.array_equal(qa[:, is4 == 0], qs[:, is4 == 0])
    # the gather the wrong way round does not satisfy the bound
    inv_perm = np.argsort(perm)
    assert not np.all(np.abs(f16(X)[:, inv_perm] - qa * s) <= s / 2 + 1e-30)


@pytest.mark.parametrize("name", ["tiny", "q_proj_7b", "down_7b"])
def test_zero_point_partials_identity(orc, name):
    """sum(u qw) - z wsum (the zero-point term from the offline weight sum) equals the
    partials of the signed codes u - z, bit for bit."""
    cfg = synth.CONFIGS[name]
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    d = orc.quantize_layer_asym(X, W, score, cfg.nb8)
    rows = (0, min(cfg.M, 24))
    Pz = orc.block_partials_zero_point(d["qa"], d["u4"], d["za"], d["qw"], d["wsum"], d["flags"], rows)
    Pq = orc.block_partials(d["qa"], d["qw"], rows)
    assert np.array_equal(Pz, Pq)
    assert np.abs(Pq).max() <= 127 * 7 * 128


@pytest.mark.parametrize("nb8", [0, 1, 4])
def test_asym_dequantize_then_matmul(orc, nb8):
    """The epilogue over the asymmetric partials equals a float64 matmul of the
    dequantized operands s (u - z) and s_w q_w."""
    X, W, score, _ = small_layer(24, 512, 40, 23, nb8)
    d = orc.quantize_layer_asym(X, W, score, nb8)
    P = orc.block_partials(d["qa"], d["qw"])
    y32, Y16, ye = orc.epilogue(P, d["sa"], d["sw16"])
    blk = np.arange(512) // 128
    A = d["qa"].astype(np.float64) * d["sa"].astype(np.float64)[:, blk]
    B = d["qw"].astype(np.float64) * f16(d["sw16"])[:, blk]
    ref, mag = A @ B.T, np.abs(A) @ np.abs(B).T
    assert np.all(np.abs(ye - ref) <= 1e-12 * mag + 1e-300)
    assert np.array_equal(Y16, y32.astype(np.float16).view(np.uint16))


def test_asym_brute_force_tiny(orc):
    """M = 3, K = 256 (one 4-bit and one 8-bit block): range, step, zero point and
    every code by exact rational arithmetic."""
    X, W, score, _ = small_layer(3, 256, 4, 53, 1)
    d = orc.quantize_layer_asym(X, W, score, 1)
    perm = sorted(range(256), key=lambda k: (float(score[k]), k))
    xv = f16(X)
    for m in range(3):
        blk = [xv[m, perm[k]] for k in range(128)]      # block 0 is the 4-bit one
        lo, hi = min(min(blk), 0.0), max(max(blk), 0.0)
        d_ = Fraction(hi) - Fraction(lo)
        s = float(np.float32(np.float32(hi) - np.float32(lo)) / np.float32(15))
        assert d["sa"][m, 0] == np.float32(s)
        zt = -Fraction(lo) * 15 / d_
        if not near_half(zt):
            assert d["za"][m, 0] == nearest(zt)
        z = int(d["za"][m, 0])
        for k in range(128):
            t = Fraction(blk[k]) * 15 / d_
            if not near_half(t):
                u = min(15, max(0, nearest(t) + z))
                assert d["u4"][m, k] == u, (m, k)
                assert d["qa"][m, k] == u - z


def test_asym_error_against_unquantized(orc):
    """On the planted-outlier 7B layer the asymmetric 4-bit blocks (finer step)
    give a smaller error against the unquantized product X W^T than the symmetric
    ones, with everything else equal."""
    cfg = synth.CONFIGS["q_proj_7b"]
    X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
    ref = f16(X) @ f16(W).T
    ys = orc.reference(X, W, score, cfg.nb8)["yexact"]
    d = orc.quantize_layer_asym(X, W, score, cfg.nb8)
    P = orc.block_partials(d["qa"], d["qw"])
    _, _, ya = orc.epilogue(P, d["sa"], d["sw16"])
    es = np.sqrt(np.mean((ys - ref) ** 2))
    ea = np.sqrt(np.mean((ya - ref) ** 2))
    assert ea < es
