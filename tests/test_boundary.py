"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import w4ax_mixed_precision_amd as comet

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "comet_w4ax.h")

OK, NULL, SHAPE, ALIGN, ARG, WORKSPACE, HIP, UNSUP = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(comet_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = comet.lib()
    names = declared_functions()
    assert set(names) >= {"comet_pack_weights", "comet_quant_act", "comet_w4ax_gemm"}
    for n in names:
        assert hasattr(L, n), n
    assert set(comet.EXPORTS) == set(names)


def test_status_strings():
    L = comet.lib()
    for s in range(8):
        assert L.comet_status_string(s)
    assert L.comet_status_string(99) == b"unknown status"
    assert comet.version().startswith("comet-w4ax")


A = 1 << 20          # a fake, 16-byte aligned "device" address: never dereferenced
MIS = A + 4          # misaligned


def qa(X=A, M=16, K=512, ldx=512, perm=A, nb8=1, Xq=A, xs=A):
    return comet.lib().comet_quant_act(X, M, K, ldx, perm, nb8, Xq, xs, None)


def gm(Xq=A, xs=A, Wq=A, ws=A, wsum=A, nb8=1, M=16, N=512, K=512, Y=A, ldy=512,
       work=None, wbytes=0):
    return comet.lib().comet_w4ax_gemm(Xq, xs, Wq, ws, wsum, nb8, M, N, K, Y, ldy, work, wbytes,
                                       None)


def gp(Xq=A, xs=A, Wq=A, ws=A, wsum=A, nb8=1, M=16, N=512, K=512, m0=0, mc=16, P=A):
    return comet.lib().comet_w4ax_gemm_partials(Xq, xs, Wq, ws, wsum, nb8, M, N, K, m0, mc, P,
                                                None)


def qf(X=A, M=16, K=512, ldx=512, perm=A, nb8=1, Xq=A, xs=A):
    return comet.lib().comet_quant_act_fp6(X, M, K, ldx, perm, nb8, Xq, xs, None)


def gf(Xq=A, xs=A, Wq=A, ws=A, nb8=1, M=16, N=512, K=512, Y=A, ldy=512, work=A, wbytes=1 << 40):
    return comet.lib().comet_w4ax_gemm_fp6(Xq, xs, Wq, ws, nb8, M, N, K, Y, ldy, work, wbytes, None)


def gfp(Xq=A, xs=A, Wq=A, ws=A, nb8=1, M=16, N=512, K=512, m0=0, mc=16, P=A, cap=0, work=A, wbytes=1 << 40):
    return comet.lib().comet_w4ax_gemm_fp6_partials(Xq, xs, Wq, ws, nb8, M, N, K, m0, mc, P, cap, work, wbytes,
                                                    None)


def test_fp6_workspace_bounds_and_noalloc_limit():
    """Split plans hold at most two waves of runs (1024 partial tiles of
    64 KiB, plus the counters), over a sweep of shapes; the allocation-free
    call's fixed scratch holds every one-wave plan (the 7B layers, the 70B
    decode shapes on this layout) and rejects a larger one with
    COMET_ERR_WORKSPACE before any HIP call."""
    L = comet.lib()
    wb = L.comet_w4ax_gemm_fp6_workspace_bytes
    worst = 0
    for M in (1, 16, 64, 100, 128, 256, 384, 512, 1024, 2048, 4096):
        for N in (128, 512, 1024, 2048, 4096, 5120, 8192, 10240, 11008, 12800, 28672):
            for K in (128, 512, 1024, 4096, 8192, 11008, 28672):
                nb = K // 128
                for nb8 in {0, nb // 4, nb}:
                    worst = max(worst, wb(M, N, K, nb8))
    assert 0 < worst <= 256 + 1024 * 128 * 128 * 4
    for M, N, K, nb8 in ((128, 4096, 4096, 4), (1024, 4096, 11008, 22), (64, 10240, 8192, 7)):
        assert 0 < wb(M, N, K, nb8) <= comet.NOALLOC_SCRATCH_BYTES
    M, N, K, nb8 = 256, 12800, 28672, 0                     # 200 tiles x 5 runs: 62.5 MiB
    assert wb(M, N, K, nb8) > comet.NOALLOC_SCRATCH_BYTES
    assert L.comet_w4ax_gemm_fp6_noalloc(A, A, A, A, nb8, M, N, K, A, N, None) == WORKSPACE


def test_fp6_workspace_contract():
    """The FP6 GEMM's workspace: a function of the shape only (no device
    needed), none for grids of a wave of whole tiles or more (the 70B prefill
    layers, the 7B up/gate layer's 688 tiles) or where splitting does not pay
    (short K, or a grid close to a wave), the split runs' partial tiles
    otherwise (q_proj_7b: 32 tiles x 8 runs; down_7b: 256 x 2); a missing,
    small or misaligned workspace is rejected before any HIP call."""
    L = comet.lib()
    wb = L.comet_w4ax_gemm_fp6_workspace_bytes
    assert wb(4096, 8192, 28672, 67) == 0 and wb(4096, 28672, 8192, 7) == 0 and wb(1024, 11008, 4096, 4) == 0
    tile = 128 * 128 * 4
    assert wb(128, 4096, 4096, 4) == 256 + 32 * 8 * tile
    assert wb(1024, 4096, 11008, 22) == 256 + 256 * 2 * tile
    assert wb(16, 512, 512, 1) == 0 and wb(384, 12800, 1024, 2) == 0        # splitting would not pay
    for M, N, K, nb8 in ((128, 4096, 4096, 4), (1024, 4096, 11008, 22), (64, 10240, 8192, 7)):
        need = wb(M, N, K, nb8)
        assert need > 0 and need % 16 == 0, (M, N, K)
        assert comet.fp6_workspace_bytes(M, N, K, nb8) == need
        assert gf(M=M, N=N, K=K, nb8=nb8, ldy=N, work=None, wbytes=0) == NULL
        assert gf(M=M, N=N, K=K, nb8=nb8, ldy=N, wbytes=need - 1) == WORKSPACE
        assert gf(M=M, N=N, K=K, nb8=nb8, ldy=N, work=MIS, wbytes=need) == ALIGN
        assert gfp(M=M, N=N, K=K, nb8=nb8, mc=1, work=None, wbytes=0) == NULL
    assert wb(16, 512, 500, 1) == 0 and wb(0, 512, 512, 1) == 0 and wb(16, 512, 512, 9) == 0


def test_fp6_rejections():
    assert qf(X=None) == NULL and qf(Xq=None) == NULL and qf(M=0) == SHAPE
    assert qf(ldx=511) == SHAPE and qf(nb8=5) == ARG and qf(Xq=MIS) == ALIGN
    assert gf(Xq=None) == NULL and gf(Wq=None) == NULL and gf(ws=None) == NULL and gf(Y=None) == NULL
    assert gf(M=0) == SHAPE and gf(K=100) == SHAPE and gf(ldy=500) == SHAPE
    assert gf(nb8=5) == ARG and gf(N=200, ldy=200) == UNSUP
    assert gf(Wq=MIS) == ALIGN and gf(Y=MIS) == ALIGN and gf(xs=MIS) == ALIGN
    assert gf(M=1 << 20, N=1 << 12, ldy=1 << 12) == UNSUP
    assert gfp(P=None) == NULL and gfp(m0=10, mc=7) == SHAPE and gfp(P=MIS) == ALIGN and gfp(cap=-1) == ARG
    L = comet.lib()
    assert L.comet_xq_fp6_bytes(16, 512, 1) == comet.xq_fp6_bytes(16, 512, 1) == 16 * (96 * 3 + 128)
    assert L.comet_wq_fp6_bytes(256, 512, 1) == comet.wq_fp6_bytes(256, 512, 1) == 256 * (96 * 3 + 64)
    assert L.comet_xq_fp6_bytes(16, 500, 1) == 0 and L.comet_wq_fp6_bytes(256, 512, 9) == 0
    p = ctypes.c_void_p(A)
    assert L.comet_repack_weights_fp6(None, 128, 256, 0, p) == NULL
    assert L.comet_repack_weights_fp6(p, 128, 200, 0, p) == SHAPE
    assert L.comet_repack_weights_fp6(p, 128, 256, 3, p) == ARG
    assert L.comet_repack_weights_fp6(p, 100, 256, 0, p) == UNSUP


def test_quant_act_rejections():
    assert qa(X=None) == NULL and qa(perm=None) == NULL and qa(Xq=None) == NULL
    assert qa(xs=None) == NULL
    assert qa(M=0) == SHAPE and qa(K=100) == SHAPE and qa(K=0) == SHAPE
    assert qa(ldx=511) == SHAPE
    assert qa(nb8=-1) == ARG and qa(nb8=5) == ARG
    assert qa(X=MIS) == ALIGN and qa(perm=MIS) == ALIGN and qa(Xq=MIS) == ALIGN
    assert qa(xs=MIS) == ALIGN


def test_gemm_rejections():
    assert gm(Xq=None) == NULL and gm(Y=None) == NULL and gm(wsum=None) == NULL
    assert gm(M=0) == SHAPE and gm(N=0) == SHAPE and gm(K=384 + 1) == SHAPE
    assert gm(ldy=500) == SHAPE
    assert gm(nb8=5) == ARG and gm(nb8=-2) == ARG
    assert gm(N=200, ldy=200) == UNSUP
    assert gm(Wq=MIS) == ALIGN and gm(Y=MIS) == ALIGN and gm(ws=MIS) == ALIGN
    assert gm(M=1 << 20, N=1 << 12, ldy=1 << 12) == UNSUP       # M*N beyond int32


def test_gemm_workspace_contract():
    L = comet.lib()
    for M, N, K in ((1, 8192, 8192), (16, 28672, 8192), (4096, 8192, 28672), (16, 512, 512)):
        need = L.comet_w4ax_gemm_workspace_bytes(M, N, K, 1)
        if need:
            assert gm(M=M, N=N, K=K, ldy=N, work=None) == NULL
            assert gm(M=M, N=N, K=K, ldy=N, work=A, wbytes=need - 1) == WORKSPACE
            assert gm(M=M, N=N, K=K, ldy=N, work=MIS, wbytes=need) == ALIGN
    assert L.comet_w4ax_gemm_workspace_bytes(0, 512, 512, 0) == 0


def test_partials_rejections():
    assert gp(P=None) == NULL
    assert gp(m0=-1) == SHAPE and gp(mc=0) == SHAPE and gp(m0=10, mc=7) == SHAPE
    assert gp(P=MIS) == ALIGN


def test_pack_rejections():
    W = np.zeros((128, 256), np.uint16)
    s = np.zeros(256, np.float32)
    with pytest.raises(comet.CometError) as e:
        comet.comet_pack_weights(np.zeros((128, 200), np.uint16), np.zeros(200, np.float32), 0)
    assert e.value.status == SHAPE
    with pytest.raises(comet.CometError) as e:
        comet.comet_pack_weights(W, s, 3)
    assert e.value.status == ARG
    with pytest.raises(comet.CometError) as e:
        comet.comet_pack_weights(np.zeros((100, 256), np.uint16), s, 0)
    assert e.value.status == UNSUP
    bad = s.copy()
    bad[3] = np.inf
    with pytest.raises(comet.CometError) as e:
        comet.comet_pack_weights(W, bad, 0)
    assert e.value.status == ARG
    Wn = W.copy()
    Wn[5, 7] = 0x7E00                      # NaN weight
    with pytest.raises(comet.CometError) as e:
        comet.comet_pack_weights(Wn, s, 0)
    assert e.value.status == ARG
    L = comet.lib()
    p = ctypes.c_void_p(A)
    assert L.comet_pack_weights(None, 128, 256, p, 0, p, p, p, p, p) == NULL


def test_rmsnorm_quant_rejections():
    """Fused normalization + quantization: every check before any HIP call."""
    L = comet.lib()
    a = 4096          # 16-byte aligned fake device addresses; never dereferenced
    for f in (L.comet_rmsnorm_quant_act, L.comet_rmsnorm_quant_act_fp6):
        ok = (a, 4, 256, 256, a, 1e-5, a, 1, a, a, None)
        def call(**kw):
            args = list(ok)
            for i, v in kw.items():
                args[int(i[1:])] = v
            return f(*args)
        assert call(a4=None) == NULL and call(a0=None) == NULL and call(a6=None) == NULL
        assert call(a8=None) == NULL and call(a9=None) == NULL
        assert call(a1=0) == SHAPE and call(a2=200) == SHAPE and call(a3=128) == SHAPE
        assert call(a7=3) == ARG and call(a7=-1) == ARG
        for eps in (0.0, -1e-5, float("inf"), float("nan")):
            assert call(a5=eps) == ARG, eps
        assert call(a4=a + 2) == ALIGN and call(a0=a + 8) == ALIGN


def test_rmsnorm_rejections():
    L = comet.lib()
    a = 4096
    f = L.comet_rmsnorm
    assert f(None, 2, 64, 64, a, 1e-5, a, 64, None) == NULL
    assert f(a, 2, 64, 64, None, 1e-5, a, 64, None) == NULL
    assert f(a, 2, 64, 64, a, 1e-5, None, 64, None) == NULL
    assert f(a, 0, 64, 64, a, 1e-5, a, 64, None) == SHAPE
    assert f(a, 2, 0, 64, a, 1e-5, a, 64, None) == SHAPE
    assert f(a, 2, 64, 63, a, 1e-5, a, 64, None) == SHAPE
    assert f(a, 2, 64, 64, a, 1e-5, a, 63, None) == SHAPE
    assert f(a, 2, 64, 64, a, 0.0, a, 64, None) == ARG
    assert f(a, 2, 64, 64, a, float("nan"), a, 64, None) == ARG
    assert f(a + 1, 2, 64, 64, a, 1e-5, a, 64, None) == ALIGN


def test_swiglu_quant_rejections():
    """Fused SwiGLU + quantization: every check before any HIP call."""
    L = comet.lib()
    a = 4096
    for f in (L.comet_swiglu_quant_act, L.comet_swiglu_quant_act_fp6):
        ok = (a, a, 4, 256, 512, a, 1, a, a, None)
        def call(**kw):
            args = list(ok)
            for i, v in kw.items():
                args[int(i[1:])] = v
            return f(*args)
        for i in (0, 1, 5, 7, 8):
            assert call(**{f"a{i}": None}) == NULL, i
        assert call(a2=0) == SHAPE and call(a3=200) == SHAPE and call(a3=0) == SHAPE and call(a4=255) == SHAPE
        assert call(a6=3) == ARG and call(a6=-1) == ARG
        assert call(a0=a + 2) == ALIGN and call(a1=a + 8) == ALIGN and call(a7=a + 4) == ALIGN


def test_swiglu_rejections():
    L = comet.lib()
    a = 4096
    f = L.comet_swiglu
    assert f(None, a, 2, 64, 64, a, 64, None) == NULL
    assert f(a, None, 2, 64, 64, a, 64, None) == NULL
    assert f(a, a, 2, 64, 64, None, 64, None) == NULL
    assert f(a, a, 0, 64, 64, a, 64, None) == SHAPE
    assert f(a, a, 2, 0, 64, a, 64, None) == SHAPE
    assert f(a, a, 2, 64, 63, a, 64, None) == SHAPE
    assert f(a, a, 2, 64, 64, a, 63, None) == SHAPE
    assert f(a + 1, a, 2, 64, 64, a, 64, None) == ALIGN
    assert f(a, a + 1, 2, 64, 64, a, 64, None) == ALIGN
    assert f(a, a, 2, 64, 64, a + 1, 64, None) == ALIGN


def test_permute_channels():
    v = (np.arange(300, dtype=np.uint16) * 7) % 65000
    perm = np.random.default_rng(3).permutation(300).astype(np.int32)
    assert np.array_equal(comet.comet_permute_channels(v, perm), v[perm])
    L = comet.lib()
    bad = perm.copy()
    bad[5] = 300
    out = np.empty(300, np.uint16)
    P = lambda x: x.ctypes.data_as(ctypes.c_void_p)
    assert L.comet_permute_channels(P(v), P(bad), 300, P(out)) == ARG
    assert L.comet_permute_channels(P(v), P(perm), 0, P(out)) == SHAPE
    assert L.comet_permute_channels(None, P(perm), 300, P(out)) == NULL


def qaa(X=A, M=16, K=512, ldx=512, perm=A, nb8=1, Xq=A, xs=A, xz=A):
    return comet.lib().comet_quant_act_asym(X, M, K, ldx, perm, nb8, Xq, xs, xz, None)


def gma(Xq=A, xs=A, xz=A, Wq=A, ws=A, wsum=A, nb8=1, M=16, N=512, K=512, Y=A, ldy=512):
    return comet.lib().comet_w4ax_gemm_asym(Xq, xs, xz, Wq, ws, wsum, nb8, M, N, K, Y, ldy, None, 0, None)


def gpa(Xq=A, xs=A, xz=A, Wq=A, ws=A, wsum=A, nb8=1, M=16, N=512, K=512, m0=0, mc=16, P=A):
    return comet.lib().comet_w4ax_gemm_asym_partials(Xq, xs, xz, Wq, ws, wsum, nb8, M, N, K, m0, mc, P, None)


def test_asym_rejections():
    """The asymmetric-code calls: the checks of their symmetric forms plus the zero points."""
    assert qaa(xz=None) == NULL and qaa(X=None) == NULL and qaa(xs=None) == NULL
    assert qaa(M=0) == SHAPE and qaa(K=100) == SHAPE and qaa(ldx=511) == SHAPE
    assert qaa(nb8=5) == ARG and qaa(nb8=-1) == ARG
    assert qaa(xz=MIS) == ALIGN and qaa(Xq=MIS) == ALIGN
    assert gma(xz=None) == NULL and gma(Y=None) == NULL and gma(wsum=None) == NULL
    assert gma(xz=MIS) == ALIGN and gma(Wq=MIS) == ALIGN
    assert gma(M=0) == SHAPE and gma(ldy=500) == SHAPE and gma(nb8=5) == ARG
    assert gma(N=200, ldy=200) == UNSUP
    assert gpa(xz=None) == NULL and gpa(P=None) == NULL and gpa(xz=MIS) == ALIGN
    assert gpa(m0=-1) == SHAPE and gpa(m0=10, mc=7) == SHAPE


def test_x_zero_bytes():
    L = comet.lib()
    assert L.comet_x_zero_bytes(1, 512) == 4 * 16
    assert L.comet_x_zero_bytes(17, 8192) == 64 * 32
    assert L.comet_x_zero_bytes(4096, 28672) == 224 * 4096
    assert L.comet_x_zero_bytes(0, 512) == 0 and L.comet_x_zero_bytes(16, 100) == 0


def test_qoq_rejections():
    L = comet.lib()

    def pq(W=A, N=128, K=256, sc=A, perm=A, Wu=A, s1=A, s2z=A):
        return L.comet_pack_weights_qoq(W, N, K, sc, perm, Wu, s1, s2z)

    def qt(X=A, M=16, K=512, ldx=512, perm=A, Xq=A, xs=A):
        return L.comet_quant_act_token_i8(X, M, K, ldx, perm, Xq, xs, None)

    def gq(Xq=A, xs=A, Wu=A, s2z=A, s1=A, M=16, N=512, K=512, Y=A, ldy=512):
        return L.comet_w4a8_qoq_gemm(Xq, xs, Wu, s2z, s1, M, N, K, Y, ldy, None)

    def gqp(Xq=A, xs=A, Wu=A, s2z=A, s1=A, M=16, N=512, K=512, P=A):
        return L.comet_w4a8_qoq_gemm_products(Xq, xs, Wu, s2z, s1, M, N, K, P, None)

    assert pq(W=None) == NULL and pq(s2z=None) == NULL
    assert pq(K=100) == SHAPE and pq(N=0) == SHAPE and pq(N=96) == UNSUP
    assert qt(X=None) == NULL and qt(xs=None) == NULL
    assert qt(M=0) == SHAPE and qt(K=100) == SHAPE and qt(ldx=500) == SHAPE
    assert qt(K=33024, ldx=33024) == UNSUP and qt(Xq=MIS) == ALIGN
    assert gq(Y=None) == NULL and gq(s1=None) == NULL
    assert gq(M=0) == SHAPE and gq(ldy=500) == SHAPE and gq(K=100) == SHAPE
    assert gq(N=200, ldy=200) == UNSUP and gq(K=33024) == UNSUP
    assert gq(M=1 << 20, N=1 << 12, ldy=1 << 12) == UNSUP
    assert gq(Wu=MIS) == ALIGN and gq(Y=MIS) == ALIGN and gq(s2z=MIS) == ALIGN
    assert gqp(P=None) == NULL and gqp(P=MIS) == ALIGN and gqp(N=96) == UNSUP


def test_kv4_rejections():
    L = comet.lib()

    def kq(X=A, ntok=4, H=8, d=128, ldx=1024, pos=0, tcap=16, codes=A, step=A, zero=A):
        return L.comet_kv4_quantize(X, ntok, H, d, ldx, pos, tcap, codes, step, zero, None)

    def ka(q=A, kc=A, ks=A, kz=A, vc=A, vs=A, vz=A, Hq=8, group=2, d=128, T=300, tcap=300, out=A, ws=A,
           wsb=1 << 20):
        return L.comet_kv4_attention(q, kc, ks, kz, vc, vs, vz, Hq, group, d, T, tcap, out, ws, wsb, None)

    assert kq(X=None) == NULL and kq(zero=None) == NULL and kq(codes=None) == NULL
    assert kq(ntok=0) == SHAPE and kq(H=0) == SHAPE and kq(ldx=1000) == SHAPE and kq(pos=-1) == SHAPE
    assert kq(pos=13) == SHAPE and kq(ntok=17) == SHAPE
    assert kq(d=96, ldx=768) == UNSUP and kq(d=4, ldx=32) == UNSUP and kq(d=1024, ldx=8192) == UNSUP
    assert kq(X=MIS) == ALIGN and kq(ldx=1028) == ALIGN and kq(step=MIS) == ALIGN
    assert ka(out=None) == NULL and ka(ws=None) == NULL and ka(vz=None) == NULL
    assert ka(Hq=0) == SHAPE and ka(group=0) == SHAPE and ka(group=3) == SHAPE
    assert ka(T=0) == SHAPE and ka(tcap=299) == SHAPE
    assert ka(d=100) == UNSUP and ka(d=1024) == UNSUP
    assert ka(wsb=0) == WORKSPACE
    assert ka(wsb=L.comet_kv4_attention_workspace_bytes(8, 128, 300) - 1) == WORKSPACE
    assert ka(q=MIS) == ALIGN and ka(ws=MIS) == ALIGN and ka(kz=MIS) == ALIGN
    assert L.comet_kv4_attention_workspace_bytes(8, 128, 300) == 8 * 2 * 130 * 4
    assert L.comet_kv4_attention_workspace_bytes(512, 128, 4096) == 512 * 16 * 130 * 4
    assert L.comet_kv4_attention_workspace_bytes(0, 128, 1) == 0
    assert L.comet_kv4_attention_workspace_bytes(4, 96, 1) == 0

    def kv(Tkv=A, Tmax=300, tcap=300, q=A, Hq=8, group=2, d=128, wsb=1 << 20):
        return L.comet_kv4_attention_varlen(q, A, A, A, A, A, A, Hq, group, d, Tkv, Tmax, tcap, A, A, wsb, None)

    assert kv(Tkv=None) == NULL and kv(q=None) == NULL
    assert kv(Tmax=0) == SHAPE and kv(tcap=299) == SHAPE and kv(group=3) == SHAPE
    assert kv(d=100) == UNSUP
    assert kv(wsb=L.comet_kv4_attention_workspace_bytes(8, 128, 300) - 1) == WORKSPACE
    assert kv(Tkv=A + 2) == ALIGN and kv(q=MIS) == ALIGN


def qq(X=A, M=16, K=512, ldx=512, perm=A, nb8=1, nf=128, Xq=A, xs=A, Xf=A):
    return comet.lib().comet_quant_act_quik_fp6(X, M, K, ldx, perm, nb8, nf, Xq, xs, Xf, None)


def gq(Xq=A, xs=A, Wq=A, ws=A, nb8=1, Xf=A, Wf=A, nf=128, M=16, N=512, K=512, Y=A, ldy=512, work=A,
       wbytes=1 << 40):
    return comet.lib().comet_w4ax_gemm_quik_fp6(Xq, xs, Wq, ws, nb8, Xf, Wf, nf, M, N, K, Y, ldy, work, wbytes,
                                                None)


def test_quik_rejections():
    """QUIK's split: n_fp16 a multiple of 128 leaving a quantized block, nb8
    within the quantized blocks; the fp16 operands required only when
    n_fp16 > 0; every check before any HIP call."""
    assert qq(X=None) == NULL and qq(Xf=None) == NULL and qq(M=0) == SHAPE and qq(ldx=500) == SHAPE
    assert qq(nf=100) == ARG and qq(nf=512) == ARG and qq(nf=-128) == ARG and qq(nb8=4) == ARG
    assert qq(Xf=MIS) == ALIGN and qq(Xq=MIS) == ALIGN
    assert gq(Xf=None) == NULL and gq(Wf=None) == NULL and gq(Y=None) == NULL
    assert gq(nf=64) == ARG and gq(nf=512) == ARG and gq(nb8=4) == ARG and gq(K=500) == SHAPE
    assert gq(M=0) == SHAPE and gq(ldy=500) == SHAPE and gq(N=200, ldy=200) == UNSUP
    assert gq(Xf=MIS) == ALIGN and gq(Wf=MIS) == ALIGN and gq(Y=MIS) == ALIGN
    # the quantized part's workspace is that of the plain FP6 call over K - n_fp16 channels
    need = comet.lib().comet_w4ax_gemm_fp6_workspace_bytes(128, 4096, 4096 - 256, 4)
    if need:
        assert gq(M=128, N=4096, K=4096, nf=256, nb8=4, ldy=4096, wbytes=need - 1) == WORKSPACE
    L = comet.lib()
    assert L.comet_xf_bytes(17, 256) == 32 * 256 * 2 and L.comet_xf_bytes(16, 100) == 0
    p = ctypes.c_void_p(A)
    assert L.comet_pack_weights_quik(None, 128, 512, p, 128, p, p, p, p, p) == NULL
    assert L.comet_pack_weights_quik(p, 128, 500, p, 128, p, p, p, p, p) == SHAPE
    assert L.comet_pack_weights_quik(p, 128, 512, p, 512, p, p, p, p, p) == ARG
    assert L.comet_pack_weights_quik(p, 100, 512, p, 128, p, p, p, p, p) == UNSUP
