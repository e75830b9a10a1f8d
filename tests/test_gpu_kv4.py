"""GPU parity of KV4 decode attention (QoQ/QServe article, section
"KV4注意力Kernel优化"; COMET article: KV cache at 4 bits) through the C ABI
against the oracle's step 9.

The cache quantizer is compared bit for bit (codes, fp16 steps, zero points),
and slots outside the written range must stay untouched. The attention output
is compared with the oracle's float64 result on the same codes within
    |out - ref| <= 2^-11 |ref| + 2^-25 + 2^-18 vmax_h,
the fp16 rounding of the result (2^-25, half the spacing of fp16 subnormals,
bounds it below 2^-14) plus an FP32 allowance: vmax_h is the largest
dequantized value magnitude of the head, and 2^-18 vmax_h is 64 FP32 rounding
units of it, above what the FP32 sums and the exponentials of the scores
contribute (the unrounded outputs, read back from the workspace partials,
were within 1.5e-6 of the float64 result at vmax_h of about 4, a quarter of
the allowance), and far below the smallest structural mistake (one token of
4096 dropped, or a zero point off by one, moves the output by about 1e-3 and
0.1 vmax_h). It is tight enough to catch a lost-precision product: fp16 dot
products on 4-bit codes held as fp16 subnormals passed the earlier 2^-16
allowance while their unrounded error was twenty times the FP32 form's.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import pack_kv4_codes, unpack_kv4_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()
    return t


def oracle_cache(O, X16, H, d):
    """X16 [ntok, H d] -> oracle codes [H, ntok, d], steps and zeros [H, ntok]."""
    ntok = X16.shape[0]
    per_head = X16.reshape(ntok, H, d).transpose(1, 0, 2).reshape(H * ntok, d)
    u, s, z = O.kv4_quantize(np.ascontiguousarray(per_head))
    return u.reshape(H, ntok, d), s.reshape(H, ntok), z.reshape(H, ntok)


def gpu_cache(torch, comet, X16, H, d, tcap, pos=0, split=None):
    """Quantize X16 into a fresh cache at pos (in two calls when split is given)."""
    c = comet.kv4_cache(H, tcap, d)
    c["codes"].fill_(0xAB)
    c["step"].fill_(0x1234)
    c["zero"].fill_(0xCD)
    X = torch.from_numpy(X16.view(np.float16)).cuda()
    if split is None:
        comet.comet_kv4_quantize(X, c, pos)
    else:
        comet.comet_kv4_quantize(X[:split], c, pos)
        comet.comet_kv4_quantize(X[split:], c, pos + split)
    return c


def read_cache(c):
    H, tcap, d = c["H"], c["tcap"], c["d"]
    b = c["codes"].cpu().numpy().reshape(H, tcap, d // 2)
    s = c["step"].cpu().numpy().view(np.uint16).reshape(H, tcap)
    z = c["zero"].cpu().numpy().reshape(H, tcap)
    return b, s, z


QUANT_CASES = [  # ntok, H, d, pos, tcap
    (1, 32, 128, 7, 16), (37, 8, 128, 0, 40), (5, 4, 64, 3, 8), (3, 2, 256, 0, 3),
    (2, 3, 8, 1, 4), (70, 2, 512, 5, 80), (513, 4, 128, 0, 513)]


@pytest.mark.parametrize("ntok,H,d,pos,tcap", QUANT_CASES)
def test_kv4_quantize_bit_exact(torch, ntok, H, d, pos, tcap):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    _, K16, V16 = synth.make_kv(100 + ntok + d, ntok, H, d)
    for X16 in (K16, V16):
        X16 = X16.copy()
        if ntok > 2:                         # special vectors: all zero, all non-negative
            X16[1, :d] = 0
            X16[2, -d:] = np.abs(X16[2, -d:].view(np.float16)).view(np.uint16)
        u, s, z = oracle_cache(O, X16, H, d)
        c = gpu_cache(torch, comet, X16, H, d, tcap, pos)
        torch.cuda.synchronize()
        b, gs, gz = read_cache(c)
        w = slice(pos, pos + ntok)
        assert np.array_equal(unpack_kv4_codes(b[:, w]), u), (ntok, H, d, "codes")
        assert np.array_equal(gs[:, w], s), (ntok, H, d, "steps")
        assert np.array_equal(gz[:, w], z), (ntok, H, d, "zeros")
        outside = np.ones(tcap, bool)
        outside[w] = False
        assert (b[:, outside] == 0xAB).all() and (gs[:, outside] == 0x1234).all() and (gz[:, outside] == 0xCD).all()


def rescale16(x16, f):
    """fp16 bit patterns times f, rounded to fp16 (to nearest even)."""
    return (x16.view(np.float16).astype(np.float64) * f).astype(np.float16).view(np.uint16)


def check_attention(torch, Hq, group, d, T, seed, tcap=None, split=None, qscale=1.0, vscale=1.0):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    H = Hq // group
    tcap = T + 5 if tcap is None else tcap
    q16, K16, V16 = synth.make_kv(seed, T, H, d, Hq)
    if qscale != 1.0:
        q16 = rescale16(q16, qscale)
    if vscale != 1.0:
        V16 = rescale16(V16, vscale)
    Ku, Ks, Kz = oracle_cache(O, K16, H, d)
    Vu, Vs, Vz = oracle_cache(O, V16, H, d)
    rep = np.arange(Hq) // group
    ref = O.kv4_attention(q16, Ku[rep], Ks[rep], Kz[rep], Vu[rep], Vs[rep], Vz[rep])
    kc = gpu_cache(torch, comet, K16, H, d, tcap, 0, split)
    vc = gpu_cache(torch, comet, V16, H, d, tcap, 0, split)
    q = torch.from_numpy(q16.view(np.float16)).cuda()
    out = comet.comet_kv4_attention(q, kc, vc, T, group)
    out2 = comet.comet_kv4_attention(q, kc, vc, T, group)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), out2.cpu().numpy().view(np.uint16)), "determinism"
    # the head's largest dequantized value |s (u - z)| present in its cache,
    # formed a few heads at a time (the big cases hold ~1e8 codes)
    step = np.abs(Vs.view(np.float16).astype(np.float64))
    dev = np.empty(Vz.shape, np.float64)
    for h0 in range(0, H, 64):
        u = Vu[h0:h0 + 64].astype(np.int16)
        dev[h0:h0 + 64] = np.abs(u - Vz[h0:h0 + 64, :, None].astype(np.int16)).max(axis=-1)
    vmax = (step * dev).max(axis=1)[rep][:, None]
    tol = 2.0**-11 * np.abs(ref) + 2.0**-25 + 2.0**-18 * vmax
    err = np.abs(o - ref)
    ratio = float((err / tol).max())
    print(f"kv4 attention Hq={Hq} group={group} d={d} T={T}: max err {err.max():.3e}, "
          f"max err/tol {ratio:.3f}", flush=True)
    assert (err <= tol).all(), (Hq, group, d, T, ratio)
    return ratio


ATT_CASES = [  # Hq, group, d, T
    (4, 1, 128, 1), (8, 1, 128, 255), (8, 2, 128, 256), (16, 8, 128, 257), (32, 1, 128, 1000),
    (4, 1, 64, 513), (2, 1, 256, 300), (2, 1, 512, 70), (4, 1, 8, 33), (8, 1, 16, 700), (8, 1, 128, 4096),
    # enough heads for 512- and 1024-token chunks, each with a ragged last chunk
    (1024, 1, 64, 700), (2048, 1, 128, 1500), (2048, 2, 64, 2100), (4096, 4, 32, 1100),
    # two query heads per workgroup at every lane-slice width the launcher picks
    (8, 2, 16, 300), (8, 2, 8, 257), (4, 2, 256, 300), (4, 2, 512, 70),
    # the matrix-instruction kernel (d = 128, groups of 2 to 16): 8- and
    # 16-row query tiles, groups that are not powers of two, one token,
    # partial score tiles and value steps, 512-token chunks with one token in
    # the last
    (16, 16, 128, 300), (12, 12, 128, 33), (24, 3, 128, 1), (10, 5, 128, 257), (64, 8, 128, 1000),
    (4096, 2, 128, 513),
    # more than 16 chunks per head (the combine step's LDS path), both kernels
    (4, 1, 128, 5000), (16, 8, 128, 5000)]


@pytest.mark.parametrize("Hq,group,d,T", ATT_CASES)
def test_kv4_attention_parity(torch, Hq, group, d, T):
    check_attention(torch, Hq, group, d, T, seed=7 + T, split=(T - 1 if T > 1 else None))


SCALE_CASES = [  # Hq, group, d, T, query scale, value scale
    # a near one-hot softmax (weights from 1 down to underflow in one chunk)
    (8, 1, 128, 700, 16.0, 1.0), (4, 2, 256, 300, 16.0, 1.0),
    # value steps in the fp16 subnormal range (the outputs too: there the
    # fp16 rounding of the result, 2^-25, bounds what can be checked), and
    # near the top of fp16
    (8, 1, 128, 513, 1.0, 2.0**-18), (8, 1, 128, 513, 16.0, 2.0**-13), (4, 2, 256, 300, 1.0, 2.0**-18),
    (8, 1, 128, 300, 4.0, 2.0**12), (4, 1, 64, 300, 1.0, 2.0**-18), (8, 2, 16, 300, 1.0, 2.0**12),
    # all-zero values: every step 0, the output exactly 0
    (4, 1, 128, 300, 1.0, 0.0), (4, 2, 256, 70, 1.0, 0.0)]


@pytest.mark.parametrize("Hq,group,d,T,qs,vs", SCALE_CASES)
def test_kv4_attention_value_ranges(torch, Hq, group, d, T, qs, vs):
    """The vector kernel over value and score ranges far from N(0, 1): the
    value weights are scaled by a power of two per chunk before they are
    split into fp16 parts, which must hold from subnormal steps to steps near
    the top of fp16 and for weights that span the whole exponent range."""
    G.log(f"[kv4 ranges] Hq={Hq} group={group} d={d} T={T} qscale={qs} vscale={vs}")
    check_attention(torch, Hq, group, d, T, seed=11 + T, qscale=qs, vscale=vs)


def test_kv4_attention_bench_size(torch):
    """The measured decode workload in full: 16 sequences x 32 heads, 4096
    cached tokens, d = 128 (LLaMA-7B attention), multi-head."""
    check_attention(torch, 512, 1, 128, 4096, seed=2024, tcap=4096)


def test_kv4_attention_gqa_bench_size(torch):
    """16 sequences of LLaMA-70B's grouped-query attention: 64 query heads over
    8 kv heads each, 4096 cached tokens."""
    check_attention(torch, 1024, 8, 128, 4096, seed=2025, tcap=4096)


VARLEN_CASES = [  # Hq, group, d, T_max: the vector kernel (one and two query heads per
    # workgroup, narrow slices), the matrix kernel (256- and 512-token chunks)
    (32, 1, 128, 1000), (16, 2, 64, 700), (8, 1, 16, 300), (64, 8, 128, 1000), (256, 8, 128, 2048),
    # more than 16 chunks at T_max, fewer in the shorter heads
    (16, 1, 128, 5000)]


@pytest.mark.parametrize("Hq,group,d,Tmax", VARLEN_CASES)
def test_kv4_attention_varlen(torch, Hq, group, d, Tmax):
    """Sequences of different lengths in one call: kv head g attends to its
    first T_kv[g] slots (clamped to [0, T_max]; an empty head gives zeros).
    Each head against the oracle over its own prefix, and with every length at
    T_max the output equals comet_kv4_attention's bit for bit."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    H = Hq // group
    G.log(f"[kv4 varlen] Hq={Hq} group={group} d={d} Tmax={Tmax}")
    rng = np.random.default_rng(Hq * 131 + d + Tmax)
    # empty, one token, full, chunk edges, past T_max (clamped), negative (empty)
    special = [v for v in (0, 1, Tmax, 255, 256, 257, 511, 512, 513, Tmax + 77, -3) if v <= Tmax + 77]
    lens = rng.integers(0, Tmax + 1, size=H)
    k = min(H, len(special))
    lens[:k] = special[:k]
    q16, K16, V16 = synth.make_kv(Hq + Tmax, Tmax, H, d, Hq)
    Ku, Ks, Kz = oracle_cache(O, K16, H, d)
    Vu, Vs, Vz = oracle_cache(O, V16, H, d)
    kc = gpu_cache(torch, comet, K16, H, d, Tmax + 3)
    vc = gpu_cache(torch, comet, V16, H, d, Tmax + 3)
    q = torch.from_numpy(q16.view(np.float16)).cuda()
    Tkv = torch.from_numpy(lens.astype(np.int32)).cuda()
    out = comet.comet_kv4_attention_varlen(q, kc, vc, Tkv, Tmax, group).cpu().numpy()
    o = out.astype(np.float64)
    worst = 0.0
    for g in range(H):
        T = int(min(max(lens[g], 0), Tmax))
        hq = slice(g * group, (g + 1) * group)
        if T == 0:
            assert (out[hq].view(np.uint16) == 0).all(), f"head {g}: no tokens must give zeros"
            continue
        sel = [g] * group
        ref = O.kv4_attention(q16[hq], Ku[sel, :T], Ks[sel, :T], Kz[sel, :T], Vu[sel, :T], Vs[sel, :T], Vz[sel, :T])
        step = np.abs(Vs[g, :T].view(np.float16).astype(np.float64))
        dev = np.abs(Vu[g, :T].astype(np.int16) - Vz[g, :T, None].astype(np.int16)).max(axis=-1)
        vmax = (step * dev).max()
        tol = 2.0**-11 * np.abs(ref) + 2.0**-25 + 2.0**-18 * vmax
        err = np.abs(o[hq] - ref)
        worst = max(worst, float((err / tol).max()))
        assert (err <= tol).all(), (g, T, float((err / tol).max()))
    print(f"kv4 varlen Hq={Hq} group={group} d={d} Tmax={Tmax}: max err/tol {worst:.3f}", flush=True)
    full = torch.full((H,), Tmax, dtype=torch.int32, device="cuda")
    a = comet.comet_kv4_attention_varlen(q, kc, vc, full, Tmax, group)
    b = comet.comet_kv4_attention(q, kc, vc, Tmax, group)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "all lengths at T_max must equal the uniform call"
