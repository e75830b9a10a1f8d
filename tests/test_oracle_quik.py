"""Pins of the oracle's step 10, QUIK's fp16 outlier columns (QUIK blog,
deep-paper.org/paper/2310.09259, sections "第一步: 识别与重排" and "第二步:
前向传播 (在线)"): the highest-scoring channels stay fp16 on their own path, the
rest are quantized, and the two results are added.

Each check ties the oracle to something outside it: the plain path (nf = 0),
exact rational sums, a float64 dequantize-then-matmul, joint channel
relabelling, and the accuracy the split is for."""
from fractions import Fraction

import numpy as np
import pytest

from gen import synth


def _layer(seed, M, N, K, outliers=0.1, mult=50.0):
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, K)).astype(np.float32)
    cols = rng.permutation(K)[: int(round(outliers * K))]
    X[:, cols] *= mult
    W = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    score = np.abs(X).max(0) + rng.random(K).astype(np.float32) * 1e-3      # distinct scores
    return synth.to_fp16(X), synth.to_fp16(W), score.astype(np.float32), cols


def _f16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("nb8", [0, 1])
def test_nf0_is_the_plain_path(orc, nb8):
    X, W, score, _ = _layer(1, 8, 32, 512)
    q = orc.quik_layer(X, W, score, nb8, 0)
    r = orc.reference(X, W, score, nb8)
    assert np.array_equal(q["perm"], r["perm"]) and np.array_equal(q["flags"], r["flags"])
    assert np.array_equal(q["Y16"], r["Y16"])
    assert np.array_equal(q["yexact"], r["yexact"])


def test_split_takes_the_highest_scores(orc):
    X, W, score, _ = _layer(2, 4, 16, 1024)
    for nf in (128, 256, 512):
        perm, flags = orc.quik_split(score, 1, nf)
        assert set(perm[-nf:].tolist()) == set(np.argsort(score)[-nf:].tolist())
        assert flags.shape == ((1024 - nf) // 128,) and flags[-1] == 1 and flags[:-1].sum() == 0


def test_outlier_part_alone_is_the_exact_sum(orc):
    """With every quantized channel zero the quantized part is exactly 0, so
    yexact is the exact rational sum of the fp16 products (to binary64) and
    y32 the FP32 sum in channel order, both checked with fractions."""
    M, N, K, nf = 3, 5, 384, 128
    X, W, score, _ = _layer(3, M, N, K)
    perm, _ = orc.quik_split(score, 0, nf)
    X = X.copy()
    X[:, perm[: K - nf]] = 0
    q = orc.quik_layer(X, W, score, 0, nf)
    xs, ws = _f16(X[:, perm[K - nf:]]), _f16(W[:, perm[K - nf:]])
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xs[m], ws[n]))
            assert abs(Fraction(float(q["yexact"][m, n])) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**80)
            y = np.float32(0)
            for a, b in zip(xs[m], ws[n]):
                p = np.float32(a) * np.float32(b)
                assert Fraction(float(p)) == Fraction(float(a)) * Fraction(float(b))   # exact in FP32
                y = np.float32(y + p)
            assert q["y32"][m, n] == y


def test_dequantize_then_matmul(orc):
    """yexact = the float64 product of the dequantized quantized part plus the
    fp16 part, computed from the logical arrays."""
    M, N, K, nb8, nf = 6, 24, 768, 1, 256
    X, W, score, _ = _layer(4, M, N, K)
    q = orc.quik_layer(X, W, score, nb8, nf)
    kq = K - nf
    nbq = kq // 128
    sa = np.repeat(q["sa"].astype(np.float64), 128, axis=1)                       # [M, kq]
    sw = np.repeat(_f16(q["sw16"]), 128, axis=1)                                 # [N, kq]
    y = (q["qa"].astype(np.float64) * sa) @ (q["qw"].astype(np.float64) * sw).T
    y += _f16(q["Xf_all"]) @ _f16(q["Wf"]).T
    assert nbq == q["sa"].shape[1]
    assert np.allclose(q["yexact"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_joint_channel_relabelling(orc):
    """Relabelling the channels of X, W and the scores together leaves every
    output bit unchanged (the split follows the scores, not the labels)."""
    M, N, K, nf = 4, 16, 640, 128
    X, W, score, _ = _layer(5, M, N, K)
    q = orc.quik_layer(X, W, score, 1, nf)
    sigma = np.random.default_rng(9).permutation(K)
    q2 = orc.quik_layer(X[:, sigma], W[:, sigma], score[sigma], 1, nf)
    assert np.array_equal(q["Y16"], q2["Y16"])
    assert np.array_equal(q["yexact"], q2["yexact"])


def test_brute_force_tiny(orc):
    """Two rows, three output channels, 256 channels (128 quantized, 128 fp16):
    yexact against a rational evaluation from the codes, scales and fp16 values."""
    M, N, K, nf = 2, 3, 256, 128
    X, W, score, _ = _layer(6, M, N, K)
    q = orc.quik_layer(X, W, score, 0, nf)
    xs, ws = _f16(q["Xf_all"]), _f16(q["Wf"])
    for m in range(M):
        for n in range(N):
            P = sum(int(a) * int(b) for a, b in zip(q["qa"][m], q["qw"][n]))
            assert P == int(q["P"][m, n, 0])
            exact = Fraction(float(q["sa"][m, 0])) * Fraction(float(_f16(q["sw16"][n, 0]))) * P
            exact += sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xs[m], ws[n]))
            assert abs(Fraction(float(q["yexact"][m, n])) - exact) <= abs(exact) * Fraction(1, 2**48) + Fraction(1, 2**70)


def test_fp16_outliers_beat_their_quantized_forms(orc):
    """The point of the split: with 10% of channels x50, keeping the top
    channels in fp16 gives a smaller error against the unquantized product
    than the all-4-bit path, and than the same channels as 8-bit blocks."""
    M, N, K = 32, 64, 1024
    X, W, score, cols = _layer(7, M, N, K, outliers=0.1, mult=50.0)
    ref = _f16(X) @ _f16(W).T
    def err(y):
        return float(np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    e_quik = err(orc.quik_layer(X, W, score, 0, 128)["yexact"])
    e_w4 = err(orc.reference(X, W, score, 0)["yexact"])
    e_w8 = err(orc.reference(X, W, score, 1)["yexact"])
    assert e_quik < e_w8 < e_w4, (e_quik, e_w8, e_w4)
