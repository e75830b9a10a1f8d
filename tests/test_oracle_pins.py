"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check compares the oracle with something it does not compute the same
way: a library routine (numpy's IEEE fp16 cast, Python's sort, a float64
matmul), exact rational arithmetic, a closed form, an invariant, a brute-force
enumeration, or a hand-derived worked example (tests/golden/). The aim is that
a plausible slip anywhere in the oracle (a dropped term, a wrong sign or index,
a transposed operand, the permutation applied the wrong way round, the wrong
rounding mode) fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from gen import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")

ALL_POS_FP16 = np.arange(1, 0x7C00, dtype=np.uint16)   # every positive finite fp16


def f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def small_layer(M, K, N, seed, nb8, outliers=True):
    cfg = synth.LayerConfig("t", M, K, N, seed, x_kind="planted" if outliers else "student_t")
    X = synth.make_x(cfg)
    W = synth.make_w(cfg)
    s = synth.make_scores(cfg)
    return X, W, s, nb8


def dequant_product(d):
    """sum_k (s_x q_a)(s_w q_w) as a float64 matmul of the dequantized operands."""
    K = d["qa"].shape[1]
    blk = np.arange(K) // 128
    A = d["qa"].astype(np.float64) * d["sa"].astype(np.float64)[:, blk]
    B = d["qw"].astype(np.float64) * f16(d["sw16"])[:, blk]
    return A @ B.T, np.abs(A) @ np.abs(B).T


# --------------------------------------------------------------------------
# IEEE binary16 conversions
# --------------------------------------------------------------------------

def test_half_to_float_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.half_to_float_array(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # plus every fp16 value, every midpoint between neighbours, and nudges around them
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    extra = np.concatenate([v.astype(np.float32), mids, np.nextafter(mids, np.float32(0)),
                            np.nextafter(mids, np.float32(np.inf)), [65504, 65519.99, 65520,
                                                                    1e9, 2.0**-25, 2.0**-26]])
    f = np.concatenate([f, extra.astype(np.float32), -extra.astype(np.float32)])
    got = orc.float_to_half_array(f)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# 1. Channel order
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K,nb8", [(128, 0), (128, 1), (512, 1), (1024, 3), (4096, 4)])
def test_channel_order_against_python_sort(orc, K, nb8):
    rng = np.random.default_rng(K + nb8)
    score = rng.integers(0, 40, size=K).astype(np.float32)  # many ties
    perm, flags = orc.channel_order(score, nb8)
    ref = sorted(range(K), key=lambda k: (float(score[k]), k))
    assert perm.tolist() == ref
    assert sorted(perm.tolist()) == list(range(K))           # bijection
    assert np.all(np.diff(score[perm]) >= 0)                  # non-decreasing scores
    nb = K // 128
    assert flags.tolist() == [0] * (nb - nb8) + [1] * nb8    # 8-bit blocks last


def test_channel_order_closed_form(orc):
    # score(c) = 37 c mod 256 is a bijection of [0, 256); 37 * 173 = 1 (mod 256),
    # so the channel at sorted position k' is 173 k' mod 256.
    K = 256
    score = ((37 * np.arange(K)) % K).astype(np.float32)
    perm, flags = orc.channel_order(score, 1)
    assert perm.tolist() == [(173 * k) % K for k in range(K)]
    assert flags.tolist() == [0, 1]


def test_channel_order_rejects(orc):
    with pytest.raises(ValueError):
        orc.channel_order(np.zeros(100, np.float32), 0)      # K not a multiple of 128
    with pytest.raises(ValueError):
        orc.channel_order(np.zeros(256, np.float32), 3)      # nb8 > nb
    with pytest.raises(ValueError):
        orc.channel_order(np.zeros(256, np.float32), -1)
    s = np.zeros(256, np.float32)
    s[5] = np.nan
    with pytest.raises(ValueError):
        orc.channel_order(s, 0)


def test_outliers_land_in_int8_blocks(orc):
    cfg = synth.CONFIGS["q_proj_7b"]
    score = synth.make_scores(cfg)
    ch, _ = synth.outlier_plan(cfg)
    perm, flags = orc.channel_order(score, cfg.nb8)
    int8_channels = set(perm[(cfg.nb - cfg.nb8) * 128:].tolist())
    # every planted outlier channel (x20..x100) outranks every normal channel
    assert set(ch.tolist()) <= int8_channels


# --------------------------------------------------------------------------
# 2. Weight quantization
# --------------------------------------------------------------------------

def test_weight_scale_exhaustive(orc):
    """Every positive finite fp16 absmax: the scale is an fp16 value nearest a/7."""
    a = f16(ALL_POS_FP16)
    got = np.array([orc.weight_scale(float(x)) for x in a], dtype=np.uint16)
    s = f16(got)
    assert np.all(s > 0)
    exact = a / 7.0
    tiny = exact < 2.0 ** -25          # a/7 rounds to zero in fp16 -> smallest subnormal
    assert np.all(got[tiny] == 1)
    # nearest fp16: no other fp16 value is closer to a/7 (ties within the fp32 rounding
    # of the intermediate quotient are allowed either way)
    up = f16(got.astype(np.uint32) + 1)
    dn = f16(np.maximum(got.astype(np.int64) - 1, 0).astype(np.uint16))
    ok = tiny | ((np.abs(s - exact) <= np.abs(up - exact) * (1 + 2**-22)) &
                 (np.abs(s - exact) <= np.abs(dn - exact) * (1 + 2**-22)))
    assert np.all(ok)


def brute_nearest(v, s, qmax):
    """argmin over j in [-qmax, qmax] of |v - j s|, exact, ties to the even j."""
    v = v if isinstance(v, Fraction) else Fraction(float(v))
    s = s if isinstance(s, Fraction) else Fraction(float(s))
    best = None
    for j in range(-qmax, qmax + 1):
        d = abs(v - j * s)
        if best is None or d < best[0] or (d == best[0] and j % 2 == 0):
            best = (d, j)
    return best[1]


def test_weight_quantization_brute_force(orc):
    X, W, score, _ = small_layer(4, 256, 6, 11, 0)
    # make one group all-zero and one a single tiny value (subnormal scale)
    W = W.copy()
    W[2, :] = 0
    W[3, :] = 0
    W[3, 17] = 2  # fp16 bits 2 = 2 * 2^-24
    # a/7 = (10/7) 2^-24 rounds to the smallest subnormal, so the code -10 is clamped to -7
    W[4, 128:] = 0
    W[4, 130] = 0x800A  # -10 * 2^-24
    perm = np.arange(256, dtype=np.int32)
    qw, sw16, wsum = orc.quantize_weights(W, perm)
    wv = f16(W)
    for n in range(6):
        for b in range(2):
            s = f16(sw16[n, b])
            blk = wv[n, b * 128:(b + 1) * 128]
            if np.all(blk == 0):
                assert sw16[n, b] == 0 and np.all(qw[n, b * 128:(b + 1) * 128] == 0)
                continue
            for k in range(128):
                assert qw[n, b * 128 + k] == brute_nearest(blk[k], s, 7)
            assert wsum[n, b] == int(qw[n, b * 128:(b + 1) * 128].astype(np.int64).sum())
            # the absmax element lands on +-7
            kk = int(np.argmax(np.abs(blk)))
            if s > 2.0 ** -24:
                assert abs(int(qw[n, b * 128 + kk])) == 7
    assert sw16[3, 0] == 1 and qw[3, 17] == 2     # 2 * 2^-24 / 2^-24 = 2
    assert sw16[4, 1] == 1 and qw[4, 130] == -7   # clamped


def test_weight_round_trip_bound(orc):
    cfg = synth.CONFIGS["q_proj_7b"]
    W = synth.make_w(cfg)[:256]
    score = synth.make_scores(cfg)
    perm, _ = orc.channel_order(score, cfg.nb8)
    qw, sw16, wsum = orc.quantize_weights(W, perm)
    wp = f16(W)[:, perm]
    s = f16(sw16)[:, np.arange(cfg.K) // 128]
    err = np.abs(wp - qw * s)
    assert np.all(err <= s / 2 * (1 + 2**-20))
    assert np.all(np.abs(qw) <= 7)
    assert np.array_equal(wsum, qw.reshape(256, -1, 128).astype(np.int64).sum(-1))


# --------------------------------------------------------------------------
# 3. Activation quantization
# --------------------------------------------------------------------------

def _correctly_rounded_f32(x: Fraction, got: float) -> bool:
    g = Fraction(float(np.float32(got)))
    lo = Fraction(float(np.nextafter(np.float32(got), np.float32(-np.inf))))
    hi = Fraction(float(np.nextafter(np.float32(got), np.float32(np.inf))))
    d = abs(g - x)
    if d > abs(lo - x) or d > abs(hi - x):
        return False
    if d == abs(lo - x) or d == abs(hi - x):       # exact tie: even significand wins
        return (np.float32(got).view(np.uint32) & 1) == 0
    return True


@pytest.mark.parametrize("qmax", [7, 127])
def test_act_scale_exhaustive(orc, qmax):
    """Every positive finite fp16 absmax: inv = qmax/a and s = a/qmax correctly rounded,
    s * qmax within one fp32 ulp of a, and the absmax element itself codes to qmax."""
    a = f16(ALL_POS_FP16)
    for x in a:
        inv, s = orc.act_scale(float(x), qmax)
        fx = Fraction(float(x))
        assert _correctly_rounded_f32(Fraction(qmax) / fx, inv)
        assert _correctly_rounded_f32(fx / qmax, s)
        ulp = float(np.spacing(np.float32(x)))
        assert abs(float(s) * qmax - float(x)) <= ulp
        assert orc.act_quantize_value(float(x), inv, qmax) == qmax
        assert orc.act_quantize_value(-float(x), inv, qmax) == -qmax


@pytest.mark.parametrize("qmax", [7, 127])
def test_act_element_every_fp16(orc, qmax):
    """Every fp16 x in [-a, a] at a few absmax values: the code is a nearest integer of
    the exact t = x qmax / a up to the fp32 error of inv and of the product
    (|q - t| <= 1/2 + 2^-22 |t|), it is the nearest integer away from half-way points,
    and exact half-way products round to even."""
    allv = f16(np.arange(0, 0x7C00, dtype=np.uint16))
    for a in (7.0, 1.0, 0.3330078125, 100.0, 2.0 ** -20, 60000.0):
        inv, s = orc.act_scale(a, qmax)
        xs = allv[allv <= a]
        xs = np.concatenate([xs, -xs])
        for x in xs[:: max(1, len(xs) // 4000)]:
            q = orc.act_quantize_value(float(x), inv, qmax)
            t = Fraction(float(x)) * qmax / Fraction(a)
            assert abs(q) <= qmax
            assert abs(Fraction(q) - t) <= Fraction(1, 2) + abs(t) * Fraction(1, 2**22)
            fl = t.numerator // t.denominator
            if abs((t - fl) - Fraction(1, 2)) > abs(t) * Fraction(1, 2**21):
                assert q == (fl + 1 if t - fl > Fraction(1, 2) else fl)
            p32 = np.float32(x) * np.float32(inv)
            if float(p32) - np.floor(float(p32)) == 0.5:
                assert q % 2 == 0


def test_activation_round_trip_and_gather(orc):
    """X[m, perm[k']] ~ s_x q_a within s_x/2: catches a gather applied the wrong way."""
    cfg = synth.CONFIGS["q_proj_7b"]
    X = synth.make_x(cfg)
    score = synth.make_scores(cfg)
    perm, flags = orc.channel_order(score, cfg.nb8)
    qa, sa = orc.quantize_activations(X, perm, flags)
    xp = f16(X)[:, perm]
    s = sa.astype(np.float64)[:, np.arange(cfg.K) // 128]
    err = np.abs(xp - qa * s)
    assert np.all(err <= s / 2 + 2.0**-22 * np.abs(xp) + 1e-30)
    qmax = np.where(flags[np.arange(cfg.K) // 128] == 1, 127, 7)
    assert np.all(np.abs(qa) <= qmax[None, :])
    # each (token, block) reaches its range end at the absmax element
    assert np.all(np.abs(qa).reshape(cfg.M, cfg.nb, 128).max(-1) ==
                  np.where(flags == 1, 127, 7)[None, :])
    # and the gather in the wrong direction does not satisfy the bound
    inv_perm = np.argsort(perm)
    assert not np.all(np.abs(f16(X)[:, inv_perm] - qa * s) <= s / 2 + 1e-30)


# --------------------------------------------------------------------------
# 4-5. Partials and epilogue
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nb8", [0, 1, 2, 4])
def test_dequantize_then_matmul(orc, nb8):
    """sum_b s_x s_w P equals a float64 matmul of the dequantized operands; nb8 = 0 is
    plain W4A4 and nb8 = nb plain W4A8 (per-token per-128-group INT8 A, INT4 W)."""
    X, W, score, _ = small_layer(24, 512, 40, 21, nb8)
    d = orc.reference(X, W, score, nb8)
    ref, mag = dequant_product(d)
    assert np.all(np.abs(d["yexact"] - ref) <= 1e-12 * mag + 1e-300)
    # y32 is an fp32 sum of nb rounded terms
    nb = 4
    t = np.abs(d["sa"].astype(np.float64)[:, None, :] * f16(d["sw16"])[None, :, :] * d["P"])
    bound = (nb + 2) * 2.0**-24 * t.sum(-1) * (1 + 2**-10) + 2.0**-140
    assert np.all(np.abs(d["y32"] - d["yexact"]) <= bound)
    # Y16 is the fp16 rounding of y32 (library cast)
    assert np.array_equal(d["Y16"], d["y32"].astype(np.float16).view(np.uint16))


def test_error_bound_vs_unquantized(orc):
    """A-priori bound of the quantization error against X W^T in float64."""
    for name in ("tiny", "q_proj_7b"):
        cfg = synth.CONFIGS[name]
        X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
        rows = (0, min(cfg.M, 32))
        d = orc.reference(X, W, score, cfg.nb8, rows=rows)
        xp = f16(X)[rows[0]:rows[1]][:, d["perm"]]
        wp = f16(W)[:, d["perm"]]
        exact = xp @ wp.T
        nb = cfg.nb
        sa = d["sa"][rows[0]:rows[1]].astype(np.float64)
        sw = f16(d["sw16"])
        axb = np.abs(xp).reshape(-1, nb, 128).sum(-1)          # [m, b]
        awb = np.abs(wp).reshape(-1, nb, 128).sum(-1)          # [n, b]
        bound = (0.5 * sa @ awb.T + 0.5 * axb @ sw.T + 0.25 * 128 * sa @ sw.T
                 + 1e-6 * np.abs(xp) @ np.abs(wp).T)
        assert np.all(np.abs(d["yexact"] - exact) <= bound)


def test_error_statistics_vs_unquantized(orc):
    """Rounding to the nearest code leaves errors close to independent and uniform on
    [-s/2, s/2], so the mean squared error of y against X W^T is predicted by
    sum_k (s_x^2 / 12) w'^2 + x'^2 (s_w^2 / 12). The observed value must agree within
    a factor of two; dropping the dominant block or flipping its sign must not."""
    for name in ("tiny", "q_proj_7b"):
        cfg = synth.CONFIGS[name]
        X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
        rows = (0, min(cfg.M, 32))
        d = orc.reference(X, W, score, cfg.nb8, rows=rows)
        xp = f16(X)[rows[0]:rows[1]][:, d["perm"]]
        wp = f16(W)[:, d["perm"]]
        exact = xp @ wp.T
        nb = cfg.nb
        sa = d["sa"][rows[0]:rows[1]].astype(np.float64)
        sw = f16(d["sw16"])
        w2 = (wp ** 2).reshape(-1, nb, 128).sum(-1)           # [n, b]
        x2 = (xp ** 2).reshape(-1, nb, 128).sum(-1)           # [m, b]
        pred = ((sa ** 2) @ w2.T + x2 @ (sw ** 2).T) / 12.0
        ratio = np.mean((d["yexact"] - exact) ** 2) / np.mean(pred)
        assert 0.5 < ratio < 2.0, (name, ratio)
        tb = (sa[:, None, :] * sw[None, :, :] * d["P"])
        big = int(np.argmax(np.sqrt((tb ** 2).mean(axis=(0, 1)))))
        for wrong in (d["yexact"] - tb[:, :, big], d["yexact"] - 2 * tb[:, :, big]):
            assert np.mean((wrong - exact) ** 2) / np.mean(pred) > 4.0


def test_single_block_closed_form(orc):
    """K = 128: one term, y32 = fl(fl(s_x s_w) P) and yexact = s_x s_w P exactly."""
    X, W, score, _ = small_layer(8, 128, 16, 31, 0)
    for nb8 in (0, 1):
        d = orc.reference(X, W, score, nb8)
        sx = d["sa"][:, 0].astype(np.float64)
        sw = f16(d["sw16"][:, 0])
        P = d["P"][:, :, 0].astype(np.float64)
        assert np.array_equal(d["yexact"], sx[:, None] * sw[None, :] * P)


def test_one_hot_weights(orc):
    """One nonzero weight c per group: q_w = sign(c) 7 there, s_w = fp16(|c| / 7),
    so y is the sum over blocks of s_x q_a[k*] * 7 s_w sign(c), close to sum x[k*] c."""
    M, K, N = 6, 384, 5
    X, _, score, _ = small_layer(M, K, N, 41, 1)
    rng = np.random.default_rng(3)
    W = np.zeros((N, K), np.float32)
    picks = {}
    for n in range(N):
        for b in range(3):
            k = b * 128 + int(rng.integers(128))
            W[n, k] = rng.choice([-1, 1]) * rng.uniform(0.01, 0.05)
            picks[(n, b)] = k
    W16 = synth.to_fp16(W)
    score = np.zeros(K, np.float32)          # identity permutation
    d = orc.reference(X, W16, score, 1)
    wv, xv = f16(W16), f16(X)
    for n in range(N):
        for b in range(3):
            k = picks[(n, b)]
            assert d["qw"][n, k] == 7 * np.sign(wv[n, k])
            assert d["sw16"][n, b] == synth.to_fp16(np.float32(abs(wv[n, k])) / np.float32(7))
            assert np.count_nonzero(d["qw"][n, b * 128:(b + 1) * 128]) == 1
    for m in range(M):
        for n in range(N):
            approx = sum(xv[m, picks[(n, b)]] * wv[n, picks[(n, b)]] for b in range(3))
            tol = sum(d["sa"][m, b] / 2 * abs(wv[n, picks[(n, b)]]) * 1.001 for b in range(3))
            assert abs(d["yexact"][m, n] - approx) <= tol + 1e-12


def test_brute_force_tiny(orc):
    """M, N <= 4, K = 256: every step by enumeration with exact rationals."""
    X, W, score, _ = small_layer(3, 256, 4, 51, 1)
    d = orc.reference(X, W, score, 1)
    K, nb = 256, 2
    perm = sorted(range(K), key=lambda k: (float(score[k]), k))
    xv, wv = f16(X), f16(W)
    for m in range(3):
        for b in range(nb):
            qmax = 127 if b == 1 else 7
            blk = [xv[m, perm[b * 128 + k]] for k in range(128)]
            a = max(abs(v) for v in blk)
            s = float(np.float32(a) / np.float32(qmax))
            assert d["sa"][m, b] == np.float32(s)
            for k in range(128):
                # x * inv carries two fp32 roundings; away from half-way points the code
                # is the exact nearest integer of x * qmax / a
                t = Fraction(blk[k]) * qmax / Fraction(a)
                q = d["qa"][m, b * 128 + k]
                frac = t - (t.numerator // t.denominator)
                if abs(frac - Fraction(1, 2)) > Fraction(1, 10**5):
                    assert q == brute_nearest(t, 1, qmax), (m, b, k)
    for n in range(4):
        for b in range(nb):
            blk = [wv[n, perm[b * 128 + k]] for k in range(128)]
            s = f16(d["sw16"][n, b])
            for k in range(128):
                assert d["qw"][n, b * 128 + k] == brute_nearest(blk[k], s, 7)
    for m in range(3):
        for n in range(4):
            for b in range(nb):
                p = sum(int(d["qa"][m, b * 128 + k]) * int(d["qw"][n, b * 128 + k])
                        for k in range(128))
                assert d["P"][m, n, b] == p
            ye = sum(Fraction(float(d["sa"][m, b])) * Fraction(float(f16(d["sw16"][n, b])))
                     * int(d["P"][m, n, b]) for b in range(nb))
            assert abs(Fraction(float(d["yexact"][m, n])) - ye) <= abs(ye) * Fraction(1, 2**50)


def test_joint_permutation_invariance(orc):
    """Relabelling the channels of X, W and the scores with one permutation leaves
    every result bit-identical (scores are tie-free across block boundaries)."""
    X, W, _, _ = small_layer(16, 512, 32, 61, 1)
    score = np.random.default_rng(61).permutation(512).astype(np.float32) * 0.25
    srt = np.sort(score)
    for b in range(1, 4):    # no tie straddles a block boundary
        assert srt[128 * b - 1] != srt[128 * b]
    d0 = orc.reference(X, W, score, 1)
    pi = np.random.default_rng(5).permutation(512)
    d1 = orc.reference(X[:, pi], W[:, pi], score[pi], 1)
    for key in ("sa", "sw16", "wsum", "P", "y32", "Y16", "yexact"):
        assert np.array_equal(d0[key], d1[key]), key


def test_within_block_shuffle_invariance(orc):
    """Reordering channels inside each block changes no scale, sum, partial or output."""
    X, W, score, _ = small_layer(12, 512, 24, 71, 2)
    d0 = orc.reference(X, W, score, 2)
    rng = np.random.default_rng(9)
    perm2 = d0["perm"].copy()
    for b in range(4):
        perm2[b * 128:(b + 1) * 128] = rng.permutation(perm2[b * 128:(b + 1) * 128])
    qw, sw16, wsum = orc.quantize_weights(W, perm2)
    qa, sa = orc.quantize_activations(X, perm2, d0["flags"])
    P = orc.block_partials(qa, qw)
    y32, Y16, ye = orc.epilogue(P, sa, sw16)
    assert np.array_equal(sa, d0["sa"]) and np.array_equal(sw16, d0["sw16"])
    assert np.array_equal(wsum, d0["wsum"]) and np.array_equal(P, d0["P"])
    assert np.array_equal(Y16, d0["Y16"]) and np.array_equal(ye, d0["yexact"])


@pytest.mark.parametrize("name", ["tiny", "q_proj_7b", "down_7b"])
def test_zero_extend_equals_sign_extend(orc, name):
    """For 4-bit blocks, sum((q+8) w) - 8 sum(w) == sum(q w) exactly, every block."""
    cfg = synth.CONFIGS[name]
    X, W, score = synth.make_x(cfg, rows=min(cfg.M, 16)), synth.make_w(cfg), synth.make_scores(cfg)
    d = orc.quantize_layer(X, W[:256], score, cfg.nb8)
    P = orc.block_partials(d["qa"], d["qw"])
    Pz = orc.block_partials_zero_extend(d["qa"], d["qw"], d["wsum"], d["flags"])
    assert np.array_equal(P, Pz)


def test_zero_extend_identity_random_nibbles():
    rng = np.random.default_rng(1)
    q = rng.integers(-7, 8, size=(2000, 128))
    w = rng.integers(-7, 8, size=(2000, 128))
    lhs = ((q + 8) * w).sum(1) - 8 * w.sum(1)
    assert np.array_equal(lhs, (q * w).sum(1))


def test_partials_extremes(orc):
    """|P| <= 127 * 7 * 128 = 113792, reached by an all-max block."""
    K = 128
    X = synth.to_fp16(np.ones((2, K), np.float32))
    X[1] = synth.to_fp16(-np.ones(K, np.float32))
    W = synth.to_fp16(np.full((2, K), 0.5, np.float32))
    W[1] = synth.to_fp16(np.full(K, -0.5, np.float32))
    d = orc.reference(X, W, np.zeros(K, np.float32), 1)
    assert d["P"][:, :, 0].tolist() == [[113792, -113792], [-113792, 113792]]


# --------------------------------------------------------------------------
# Hand-derived worked examples
# --------------------------------------------------------------------------

def _expand(spec, K):
    out = np.zeros(K)
    for seg in spec:
        if "from" in seg:
            out[seg["from"]:seg["to"]] = seg["value"]
        elif seg["parity"] == "even":
            out[0::2] = seg["value"]
        elif seg["parity"] == "odd":
            out[1::2] = seg["value"]
        else:
            out[:] = seg["value"]
    return out


def test_golden_worked_examples(orc):
    ex = json.load(open(GOLDEN))["examples"]
    for e in ex:
        K = e["K"]
        X = synth.to_fp16(np.tile(_expand(e["X"], K), (e["M"], 1)))
        score = np.full(K, e["score"]["all"], np.float32)
        perm, flags = orc.channel_order(score, e["nb8"])
        exp = e["expect"]
        assert np.array_equal(perm, np.arange(K))
        qa, sa = orc.quantize_activations(X, perm, flags)
        if "flags" in exp:
            assert flags.tolist() == exp["flags"], e["name"]
        assert np.array_equal(qa[0], _expand(exp["qa"], K).astype(np.int8)), e["name"]
        sa_exp = [np.float32(1) / np.float32(127) if v == "fp32(1/127)" else v
                  for v in exp["sa"]]
        assert np.array_equal(sa[0], np.array(sa_exp, np.float32)), e["name"]
        if "W" not in e:
            continue
        W = synth.to_fp16(np.tile(_expand(e["W"], K), (e["N"], 1)))
        qw, sw16, wsum = orc.quantize_weights(W, perm)
        assert sw16[0].tolist() == exp["sw16"], e["name"]
        assert np.array_equal(qw[0], _expand(exp["qw"], K).astype(np.int8)), e["name"]
        assert wsum[0].tolist() == exp["wsum"], e["name"]
        P = orc.block_partials(qa, qw)
        assert P[0, 0].tolist() == exp["P"], e["name"]
        y32, Y16, ye = orc.epilogue(P, sa, sw16)
        if "y32" in exp:
            assert y32[0].tolist() == exp["y32"] and Y16[0].tolist() == exp["Y16"]
            assert ye[0].tolist() == exp["yexact"]
        if "P_zero_extend_raw" in exp:
            Pz = orc.block_partials_zero_extend(qa, qw, wsum, flags)
            assert Pz[0, 0, 0] + 8 * wsum[0, 0] == exp["P_zero_extend_raw"][0]


# --------------------------------------------------------------------------
# RMS normalization feeding the quantizer
# --------------------------------------------------------------------------

def _exact_sumsq(x16):
    return sum((Fraction(float(v)) ** 2 for v in x16.view(np.float16).astype(np.float64)), Fraction(0))


def test_rms_sumsq_exact_on_dyadic_rows(orc):
    """Rows of multiples of 2^-8 in [-4, 4]: the exact sum of squares is a
    binary64 value, so the statistic is that rational exactly."""
    rng = np.random.default_rng(11)
    for K in (128, 1000, 8192, 28672):
        x = (rng.integers(-1024, 1025, K) / 256.0).astype(np.float16).view(np.uint16)
        assert Fraction(orc.rms_sumsq(x)) == _exact_sumsq(x), K


def test_rms_sumsq_correctly_rounded_on_wide_rows(orc):
    """Heavy-tailed rows over many binades (subnormal to 65504): the statistic
    is the exact rational sum of squares rounded once to binary64, which
    Python's float() of a Fraction does (nearest, ties to even)."""
    rng = np.random.default_rng(12)
    for K in (512, 4096, 11008, 28672):
        x = np.clip(rng.standard_t(3, K) * 10.0 ** rng.uniform(-9, 4, K), -65504, 65504).astype(np.float16)
        x[: K // 64] = rng.choice([65504.0, -65504.0, 6.1e-5, -3e-8, 0.0], K // 64)
        x = x.view(np.uint16)
        assert orc.rms_sumsq(x) == float(_exact_sumsq(x)), K


def test_rms_sumsq_small_terms_and_ties(orc):
    """Closed forms where a binary64 running sum and the exact sum differ:
    one large square (2^30) followed by many squares each below half a unit
    in the last place of 2^30 (dropped one by one by a running sum, not by the
    exact sum); and sums that fall exactly halfway between two binary64
    values, which must round to the even neighbour."""
    big = np.float16(32768.0)                      # 2^15, square 2^30
    tiny = np.float16(2.0 ** -14)                  # square 2^-28 < 2^-23
    x = np.array([big] + [tiny] * 8191, np.float16).view(np.uint16)
    exact = Fraction(2) ** 30 + 8191 * Fraction(2) ** -28
    assert orc.rms_sumsq(x) == float(exact)
    assert orc.rms_sumsq(x) != 2.0 ** 30          # the running sum's value
    # 2^30 + 2^-23: halfway between 2^30 and 2^30 + 2^-22; the even one is 2^30
    h = np.array([big, 2.0 ** -12, 2.0 ** -12], np.float16).view(np.uint16)
    assert orc.rms_sumsq(h) == 2.0 ** 30
    # 2^30 + 2^-22 + 2^-23: halfway above an odd last bit: rounds up
    h = np.array([big, 2.0 ** -11, 2.0 ** -12, 2.0 ** -12], np.float16).view(np.uint16)
    assert orc.rms_sumsq(h) == 2.0 ** 30 + 2.0 ** -21
    # just past the midpoint: up; just short of it: down
    h = np.array([big, 2.0 ** -12, 2.0 ** -12, 2.0 ** -24], np.float16).view(np.uint16)
    assert orc.rms_sumsq(h) == 2.0 ** 30 + 2.0 ** -22
    # smallest subnormal squared, alone: 2^-48 exactly
    assert orc.rms_sumsq(np.array([1], np.uint16)) == 2.0 ** -48
    # 128-bit range: 28672 copies of 65504 (sum near 2^46.8)
    x = np.full(28672, 65504.0, np.float16).view(np.uint16)
    assert orc.rms_sumsq(x) == float(28672 * Fraction(65504) ** 2)


def test_rms_sumsq_order_free(orc):
    """The statistic does not depend on the order of the row (an exact sum
    rounded once): every shuffle gives the same bits."""
    rng = np.random.default_rng(16)
    x = np.clip(rng.standard_t(2, 4096) * 10.0 ** rng.uniform(-6, 4, 4096), -65504, 65504)
    x = x.astype(np.float16).view(np.uint16)
    base = orc.rms_sumsq(x)
    for _ in range(5):
        assert orc.rms_sumsq(rng.permutation(x)) == base


def test_rmsnorm_against_float64_formula(orc):
    """Against x / sqrt(mean(x^2) + eps) * gamma in float64 with one final
    rounding: the oracle rounds r to binary32 and forms two binary32
    products, so results agree to one fp16 step, rarely differing."""
    rng = np.random.default_rng(13)
    cfg = synth.LayerConfig("t", 64, 4096, 128, 5)
    X = synth.make_x(cfg)
    g = (1.0 + 0.2 * rng.standard_normal(4096)).astype(np.float16)
    Xn = f16(orc.rmsnorm(X, g.view(np.uint16), 1e-5))
    x = f16(X)
    ref = x / np.sqrt((x * x).mean(1, keepdims=True) + 1e-5) * g.astype(np.float64)
    ref16 = ref.astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(ref16).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(Xn - ref16) <= ulp)
    assert np.mean(Xn != ref16) < 2e-3


def test_rmsnorm_power_of_two_equivariance(orc):
    """Scaling a row by 2^j scales S by 4^j and r by 2^-j exactly (eps far
    below the rounding of S/K), so the normalized row is unchanged."""
    rng = np.random.default_rng(14)
    # magnitudes in [0.25, ~5]: every scaled copy stays a normal fp16 number
    z = rng.standard_normal((4, 2048))
    x = (np.sign(z) * (0.25 + np.abs(z))).astype(np.float16)
    g = (0.5 + rng.random(2048)).astype(np.float16).view(np.uint16)
    base = orc.rmsnorm(x.view(np.uint16), g, 1e-30)
    for j in (-3, 2, 5):
        xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float16)
        assert np.array_equal(orc.rmsnorm(xs.view(np.uint16), g, 1e-30), base), j


def test_rmsnorm_uses_gamma_per_channel(orc):
    """gamma applies per channel in the original order: swapping two gamma
    entries swaps exactly those two outputs."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((2, 512)).astype(np.float16).view(np.uint16)
    g = (0.5 + rng.random(512)).astype(np.float16)
    g2 = g.copy()
    g2[[3, 400]] = g[[400, 3]]
    a = f16(orc.rmsnorm(x, g.view(np.uint16), 1e-5))
    b = f16(orc.rmsnorm(x, g2.view(np.uint16), 1e-5))
    same = np.ones(512, bool)
    same[[3, 400]] = False
    assert np.array_equal(a[:, same], b[:, same])
    # the swapped channels follow their new weight: recomputing with the
    # swapped gamma applied by hand to the unnormalized rows moves them
    assert not np.array_equal(a[:, [3, 400]], b[:, [3, 400]])


def test_rmsnorm_rejects(orc):
    x = np.zeros((1, 128), np.uint16)
    g = np.full(128, 0x3C00, np.uint16)
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            orc.rmsnorm(x, g, eps)
    xbad = x.copy()
    xbad[0, 5] = 0x7C00
    with pytest.raises(ValueError):
        orc.rmsnorm(xbad, g, 1e-5)


def test_golden_rmsnorm_examples(orc):
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_examples.json")))["examples"]
    for e in ex:
        K, M = e["K"], e["M"]
        X = synth.to_fp16(np.full((M, K), e["X"]["all"]))
        g = np.full(K, e["gamma"]["all"])
        if "k0" in e["gamma"]:
            g[0] = e["gamma"]["k0"]
        Xn = orc.rmsnorm(X, synth.to_fp16(g), e["eps"])
        exp = e["expect"]
        assert f16(Xn)[0, 0] == exp["xn_k0"] and np.all(f16(Xn)[0, 1:] == exp["xn_rest"]), e["name"]
        perm, flags = orc.channel_order(np.zeros(K, np.float32), e["nb8"])
        qa, sa = orc.quantize_activations(Xn, perm, flags)
        assert qa[0, 0] == exp["qa_k0"] and np.all(qa[0, 1:] == exp["qa_rest"]), e["name"]
        sa_exp = np.float32(1.5) / np.float32(7) if exp["sa"] == "fp32(1.5/7)" else np.float32(exp["sa"])
        assert np.all(sa[0] == sa_exp), e["name"]


def test_rmsnorm_rounding_structure(orc):
    """The documented rounding: r = binary32 of the exactly rounded binary64
    reciprocal square root, then two binary32 products and one fp16 rounding.
    The statistic here is the exact rational sum of squares (dyadic rows, so
    the binary64 statistic is exact too); r is taken from it with 60-digit
    decimal arithmetic; the products use numpy float32."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    rng = np.random.default_rng(16)
    K = 1024
    for trial in range(6):
        x = (rng.integers(-2048, 2049, K) / 512.0).astype(np.float16)
        g = (0.5 + rng.random(K)).astype(np.float16)
        eps = 1e-5
        S = _exact_sumsq(x.view(np.uint16))
        v = Decimal(S.numerator) / Decimal(S.denominator) / Decimal(K) + Decimal(float(np.float32(eps)))
        r64 = float(Decimal(1) / v.sqrt())
        r32 = np.float32(r64)
        want = ((x.astype(np.float32) * r32) * g.astype(np.float32)).astype(np.float16)
        got = orc.rmsnorm(x.view(np.uint16)[None], g.view(np.uint16), eps)[0]
        assert np.array_equal(got, want.view(np.uint16)), trial


# --------------------------------------------------------------------------
# SwiGLU feeding the down projection's quantizer
# --------------------------------------------------------------------------

def _fp16_nearest(x: Fraction, negative: bool, tie_toward_zero: bool) -> int:
    """binary16 bits of the rational x rounded to nearest; ties go to the even
    significand, or toward zero when the caller knows the true value lies
    strictly inside the interval below |x|. Computed with exact rationals."""
    sign = 0x8000 if negative else 0
    a = abs(x)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 10, -24)
    m = a / Fraction(2) ** q
    r = m.numerator // m.denominator
    frac = m - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and not tie_toward_zero and r % 2 == 1):
        r += 1
    val = Fraction(r) * Fraction(2) ** q
    if val > 65504:
        return sign | 0x7C00
    return sign | int(np.float16(float(val)).view(np.uint16))


def _silu_mul_exact_bits(g: float, u: float) -> int:
    """fp16(silu(g) u) from 60-digit decimal arithmetic: silu(g) = g / (1 +
    e^-g) exactly as the definition reads; the product g u is exact."""
    from decimal import Decimal, localcontext
    neg = (np.signbit(g) != np.signbit(u))
    if g == 0 or u == 0:
        return 0x8000 if neg else 0
    with localcontext() as ctx:
        ctx.prec = 60
        G, U = Decimal(g), Decimal(u)
        s = 1 / (1 + (-G).exp())
        x = Fraction(G * U * s)
        # s rounds to 1 only when e^-g < 1e-60: the true |value| is then just
        # below |g u|, so a tie of g u on the fp16 grid resolves toward zero
        return _fp16_nearest(x, neg, tie_toward_zero=(s == 1))


def test_silu_mul_every_gate_value(orc):
    """Every finite fp16 gate value g with u = 1, and every 7th with u = -3:
    the oracle's binary64 evaluation equals the exact rounding of the
    definition computed with decimal arithmetic."""
    g = np.concatenate([np.arange(0, 0x7C00, dtype=np.uint16), np.arange(0x8000, 0xFC00, dtype=np.uint16)])
    got1 = orc.silu_mul(g, np.full(g.shape, 0x3C00, np.uint16))       # u = 1
    gs = g[::7]
    got3 = orc.silu_mul(gs, np.full(gs.shape, 0xC200, np.uint16))     # u = -3
    gv = g.view(np.float16).astype(np.float64)
    for i in range(g.size):
        assert got1[i] == _silu_mul_exact_bits(gv[i], 1.0), hex(int(g[i]))
    for i in range(gs.size):
        assert got3[i] == _silu_mul_exact_bits(float(gs.view(np.float16)[i]), -3.0), hex(int(gs[i]))


def test_silu_mul_random_pairs(orc):
    """Gate and up values of both signs over many binades, including fp16
    subnormal products and products near the fp16 maximum."""
    rng = np.random.default_rng(21)
    n = 20000
    g = (rng.choice([-1, 1], n) * 2.0 ** rng.uniform(-14, 7, n)).astype(np.float16)
    u = (rng.choice([-1, 1], n) * 2.0 ** rng.uniform(-14, 8, n)).astype(np.float16)
    got = orc.silu_mul(g.view(np.uint16), u.view(np.uint16))
    gv, uv = g.astype(np.float64), u.astype(np.float64)
    for i in range(n):
        want = _silu_mul_exact_bits(gv[i], uv[i])
        if (want & 0x7C00) == 0x7C00:
            continue                      # overflow: outside what a caller may pass
        assert got[i] == want, (float(gv[i]), float(uv[i]))


def test_silu_mul_ties_on_large_gates(orc):
    """Large gates, where sigma(g) rounds to 1 in binary64 and g u often lies
    exactly on an fp16 midpoint: the true value is below |g u|, so the result
    rounds toward zero, not to even. Cases are checked against the exact
    rounding, and enough of them are true ties to exercise the rule."""
    rng = np.random.default_rng(22)
    g = rng.integers(37, 2048, 3000).astype(np.float16)
    u = (rng.integers(-255, 256, 3000) / 64.0).astype(np.float16)
    got = orc.silu_mul(g.view(np.uint16), u.view(np.uint16))
    ties = 0
    for i in range(g.size):
        gu = Fraction(float(g[i])) * Fraction(float(u[i]))
        want = _silu_mul_exact_bits(float(g[i]), float(u[i]))
        if (want & 0x7C00) == 0x7C00:
            continue
        even = _fp16_nearest(gu, gu < 0, tie_toward_zero=False)
        ties += int(want != even)
        assert got[i] == want, (float(g[i]), float(u[i]))
    assert ties >= 50
    # a hand-checkable case: 1025 * 3 = 3075 sits halfway between 3074 and 3076
    assert orc.silu_mul(np.float16([1025]).view(np.uint16), np.float16([3]).view(np.uint16))[0] == \
        np.float16(3074).view(np.uint16)


def test_silu_mul_closed_forms_and_symmetry(orc):
    """silu(0) = 0 with the product's sign; sigma(g) -> 0 far below zero;
    negating u negates h exactly; for a fixed g, h is monotone in u with the
    direction of the sign of silu(g), which is that of g."""
    z = np.array([0x0000, 0x8000, 0x0000, 0x8000], np.uint16)
    u = np.float16([2.0, 2.0, -2.0, -2.0]).view(np.uint16)
    assert orc.silu_mul(z, u).tolist() == [0x0000, 0x8000, 0x8000, 0x0000]
    far = np.float16([-65504.0, -1000.0, -120.0]).view(np.uint16)
    assert orc.silu_mul(far, np.full(3, np.float16(65504.0).view(np.uint16))).tolist() == [0x8000] * 3
    rng = np.random.default_rng(23)
    g = rng.standard_normal(4000).astype(np.float16)
    uu = (rng.standard_normal(4000) * 4).astype(np.float16)
    h = orc.silu_mul(g.view(np.uint16), uu.view(np.uint16))
    hn = orc.silu_mul(g.view(np.uint16), (-uu).view(np.uint16))
    assert np.array_equal(h ^ 0x8000, hn)
    us = np.sort(uu)
    for gi in g[:20]:
        hv = f16(orc.silu_mul(np.full(us.shape, gi).view(np.uint16), us.view(np.uint16)))
        d = np.diff(hv)
        assert np.all(d >= 0) if gi >= 0 else np.all(d <= 0), float(gi)   # sign of silu(g) is that of g


def test_double_to_half_against_numpy(orc):
    """The binary64 -> binary16 rounding against numpy's direct conversion,
    on random values and on values a hair either side of fp16 midpoints
    (where a detour through binary32 would round twice)."""
    rng = np.random.default_rng(24)
    vals = list(rng.standard_normal(3000) * 2.0 ** rng.integers(-26, 17, 3000))
    mids = (np.arange(1, 0x7BFF, 37, dtype=np.uint16).view(np.float16).astype(np.float64) +
            np.arange(2, 0x7C00, 37, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2
    for m in mids:
        vals += [m, np.nextafter(m, 0.0), np.nextafter(m, np.inf), m * (1 + 2.0 ** -40), m * (1 - 2.0 ** -40)]
    vals += [65519.99, 65520.0, 2.0 ** -25, 2.0 ** -25 * (1 + 2.0 ** -30), 3 * 2.0 ** -26]
    for v in vals:
        for s in (1.0, -1.0):
            assert orc.double_to_half(s * v) == int(np.float16(s * v).view(np.uint16)), s * v


def test_swiglu_rows_and_rejects(orc):
    """Row form equals the element form; non-finite inputs and overflowing
    products are rejected."""
    rng = np.random.default_rng(25)
    G = rng.standard_normal((3, 300)).astype(np.float16).view(np.uint16)
    U = rng.standard_normal((3, 300)).astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.swiglu(G, U), orc.silu_mul(G, U))
    bad = G.copy(); bad[1, 7] = 0x7C00
    with pytest.raises(ValueError):
        orc.swiglu(bad, U)
    big = np.full((1, 128), np.float16(300.0).view(np.uint16), np.uint16)
    with pytest.raises(ValueError):
        orc.swiglu(big, big)              # 300 * 300 overflows fp16
