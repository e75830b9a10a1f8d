"""ctypes front end of the CPU oracle (comet_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product library never imports it.

Logical arrays (no GPU layout here):
  perm   int32 [K]        original channel at permuted position k'
  flags  uint8 [nb]       1 for the 8-bit blocks (the last nb8)
  qw     int8  [N, K]     weight codes in permuted order, [-7, 7]
  sw16   uint16 [N, nb]   fp16 bits of the weight scales
  wsum   int32 [N, nb]    per-group sums of qw
  qa     int8  [M, K]     activation codes in permuted order
  sa     f32   [M, nb]    activation scales
  P      int32 [rows, N, nb] exact block partials
  Xn     uint16 [M, K]    RMS-normalized activations (fp16 bits, original order)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "comet_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-fPIC", "-shared",
          "-fopenmp", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_half_to_float.restype = ctypes.c_float
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_weight_scale.restype = ctypes.c_uint16
        L.orc_weight_scale.argtypes = [ctypes.c_float]
        L.orc_act_scale.restype = None
        L.orc_act_scale.argtypes = [ctypes.c_float, I, P, P]
        L.orc_act_quantize_value.restype = I
        L.orc_act_quantize_value.argtypes = [ctypes.c_float, ctypes.c_float, I]
        L.orc_channel_order.argtypes = [I, P, I, P, P]
        L.orc_quantize_weights.argtypes = [P, I, I, P, P, P, P]
        L.orc_quantize_activations.argtypes = [P, I, I, I, P, P, P, P]
        L.orc_block_partials.argtypes = [P, P, I, I, I, I, I, P]
        L.orc_qoq_group.argtypes = [P, I, P, P]
        L.orc_kv4_code_vector.argtypes = [P, I, P, P, P]
        L.orc_kv4_quantize.argtypes = [P, I, I, P, P, P]
        L.orc_kv4_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, P]
        L.orc_qoq_quantize_weights.argtypes = [P, I, I, P, P, P, P, P, P]
        L.orc_qoq_quantize_activations.argtypes = [P, I, I, I, P, P, P]
        L.orc_qoq_gemm.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, P, P]
        L.orc_act_asym_params.argtypes = [ctypes.c_float, ctypes.c_float, P, P, P]
        L.orc_act_asym_code.argtypes = [ctypes.c_float, ctypes.c_float, I]
        L.orc_quantize_activations_asym.argtypes = [P, I, I, I, P, P, P, P, P, P]
        L.orc_block_partials_zero_point.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
        L.orc_block_partials_zero_extend.argtypes = [P, P, P, P, I, I, I, I, I, P]
        L.orc_epilogue.argtypes = [P, P, P, I, I, I, P, P, P]
        L.orc_forward_rows.argtypes = [P, I, I, I, P, P, P, P, I, I, I, P, P]
        L.orc_rms_sumsq.restype = ctypes.c_double
        L.orc_rms_sumsq.argtypes = [P, I]
        L.orc_rmsnorm_rows.argtypes = [P, I, I, I, P, ctypes.c_float, P, I]
        L.orc_double_to_half.argtypes = [ctypes.c_double]
        L.orc_double_to_half.restype = ctypes.c_uint16
        L.orc_silu_mul.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.orc_silu_mul.restype = ctypes.c_uint16
        L.orc_silu_mul_array.argtypes = [P, P, P, ctypes.c_int64]
        L.orc_silu_mul_array.restype = None
        L.orc_swiglu_rows.argtypes = [P, P, I, I, I, P, I]
        L.orc_threads.restype = I
        L.orc_set_threads.argtypes = [I]
        L.orc_set_threads.restype = None
        L.orc_half_to_float_array.restype = None
        L.orc_half_to_float_array.argtypes = [P, P, ctypes.c_int64]
        L.orc_float_to_half_array.restype = None
        L.orc_float_to_half_array.argtypes = [P, P, ctypes.c_int64]
        for f in ("orc_channel_order", "orc_quantize_weights", "orc_quantize_activations",
                  "orc_block_partials", "orc_block_partials_zero_extend", "orc_epilogue",
                  "orc_forward_rows", "orc_rmsnorm_rows"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def half_to_float(h: int) -> float:
    return lib().orc_half_to_float(int(h))


def float_to_half(f: float) -> int:
    return lib().orc_float_to_half(float(f))


def half_to_float_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.zeros(h.shape, np.float32)
    lib().orc_half_to_float_array(_p(h), _p(out), h.size)
    return out


def float_to_half_array(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.zeros(f.shape, np.uint16)
    lib().orc_float_to_half_array(_p(f), _p(out), f.size)
    return out


def weight_scale(a: float) -> int:
    return lib().orc_weight_scale(float(a))


def act_scale(a: float, qmax: int) -> tuple[float, float]:
    inv = np.zeros(1, np.float32)
    s = np.zeros(1, np.float32)
    lib().orc_act_scale(float(a), int(qmax), _p(inv), _p(s))
    return float(inv[0]), float(s[0])


def act_quantize_value(x: float, inv: float, qmax: int) -> int:
    return lib().orc_act_quantize_value(float(x), float(inv), int(qmax))


def channel_order(score: np.ndarray, nb8: int) -> tuple[np.ndarray, np.ndarray]:
    score = np.ascontiguousarray(score, dtype=np.float32)
    K = score.shape[0]
    perm = np.zeros(K, np.int32)
    flags = np.zeros(max(K // 128, 1), np.uint8)
    _check(lib().orc_channel_order(K, _p(score), int(nb8), _p(perm), _p(flags)), "channel_order")
    return perm, flags[: K // 128]


def quantize_weights(W16: np.ndarray, perm: np.ndarray):
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    N, K = W16.shape
    nb = K // 128
    qw = np.zeros((N, K), np.int8)
    sw16 = np.zeros((N, nb), np.uint16)
    wsum = np.zeros((N, nb), np.int32)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    _check(lib().orc_quantize_weights(_p(W16), N, K, _p(perm), _p(qw), _p(sw16), _p(wsum)),
           "quantize_weights")
    return qw, sw16, wsum


def quantize_activations(X16: np.ndarray, perm: np.ndarray, flags: np.ndarray):
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    M, K = X16.shape
    nb = K // 128
    qa = np.zeros((M, K), np.int8)
    sa = np.zeros((M, nb), np.float32)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    _check(lib().orc_quantize_activations(_p(X16), M, K, K, _p(perm), _p(flags), _p(qa), _p(sa)),
           "quantize_activations")
    return qa, sa


def act_asym_params(lo: float, hi: float) -> tuple[float, float, int]:
    """(inv, s, z) of a 4-bit block with range [lo, hi], lo <= 0 <= hi, lo < hi."""
    inv, s, z = ctypes.c_float(), ctypes.c_float(), ctypes.c_int()
    lib().orc_act_asym_params(lo, hi, ctypes.byref(inv), ctypes.byref(s), ctypes.byref(z))
    return inv.value, s.value, z.value


def act_asym_code(x: float, inv: float, z: int) -> int:
    return lib().orc_act_asym_code(x, inv, z)


def quantize_activations_asym(X16: np.ndarray, perm: np.ndarray, flags: np.ndarray):
    """Asymmetric 4-bit blocks (step 3b): (qa signed codes u - z, u4 stored codes,
    sa steps [M, nb], za zero points [M, nb])."""
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    M, K = X16.shape
    nb = K // 128
    qa = np.zeros((M, K), np.int8)
    u4 = np.zeros((M, K), np.uint8)
    sa = np.zeros((M, nb), np.float32)
    za = np.zeros((M, nb), np.uint8)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    _check(lib().orc_quantize_activations_asym(_p(X16), M, K, K, _p(perm), _p(flags), _p(qa), _p(u4),
                                               _p(sa), _p(za)), "quantize_activations_asym")
    return qa, u4, sa, za


def block_partials_zero_point(qa, u4, za, qw, wsum, flags, rows=None):
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    u4 = np.ascontiguousarray(u4, dtype=np.uint8)
    za = np.ascontiguousarray(za, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    wsum = np.ascontiguousarray(wsum, dtype=np.int32)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    P = np.zeros((m1 - m0, N, K // 128), np.int32)
    _check(lib().orc_block_partials_zero_point(_p(qa), _p(u4), _p(za), _p(qw), _p(wsum), _p(flags),
                                               M, N, K, m0, m1, _p(P)), "block_partials_zero_point")
    return P


def block_partials(qa: np.ndarray, qw: np.ndarray, rows: tuple[int, int] | None = None):
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    P = np.zeros((m1 - m0, N, K // 128), np.int32)
    _check(lib().orc_block_partials(_p(qa), _p(qw), M, N, K, m0, m1, _p(P)), "block_partials")
    return P


def block_partials_zero_extend(qa, qw, wsum, flags, rows=None):
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    wsum = np.ascontiguousarray(wsum, dtype=np.int32)
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    P = np.zeros((m1 - m0, N, K // 128), np.int32)
    _check(lib().orc_block_partials_zero_extend(_p(qa), _p(qw), _p(wsum), _p(flags), M, N, K,
                                                m0, m1, _p(P)), "block_partials_zero_extend")
    return P


def epilogue(P: np.ndarray, sa_rows: np.ndarray, sw16: np.ndarray):
    """(y32 [rows, N] f32, Y16 [rows, N] fp16 bits, yexact [rows, N] f64)."""
    P = np.ascontiguousarray(P, dtype=np.int32)
    sa_rows = np.ascontiguousarray(sa_rows, dtype=np.float32)
    sw16 = np.ascontiguousarray(sw16, dtype=np.uint16)
    rows, N, nb = P.shape
    y32 = np.zeros((rows, N), np.float32)
    Y16 = np.zeros((rows, N), np.uint16)
    ye = np.zeros((rows, N), np.float64)
    _check(lib().orc_epilogue(_p(P), _p(sa_rows), _p(sw16), rows, N, nb, _p(y32), _p(Y16),
                              _p(ye)), "epilogue")
    return y32, Y16, ye


def forward_rows(X16, perm, flags, qw, sw16, rows):
    """Steps 3-5 for rows [m0, m1) of X: (Y16 [rows, N], yexact [rows, N])."""
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    M, K = X16.shape
    N = qw.shape[0]
    m0, m1 = rows
    Y16 = np.zeros((m1 - m0, N), np.uint16)
    ye = np.zeros((m1 - m0, N), np.float64)
    _check(lib().orc_forward_rows(_p(X16), M, K, K, _p(np.ascontiguousarray(perm, np.int32)),
                                  _p(np.ascontiguousarray(flags, np.uint8)),
                                  _p(np.ascontiguousarray(qw, np.int8)),
                                  _p(np.ascontiguousarray(sw16, np.uint16)), N, m0, m1,
                                  _p(Y16), _p(ye)), "forward_rows")
    return Y16, ye


def rms_sumsq(x16: np.ndarray) -> float:
    """The row statistic sum of x^2 in the order comet_oracle.c defines."""
    x = np.ascontiguousarray(x16, dtype=np.uint16)
    return float(lib().orc_rms_sumsq(_p(x), x.size))


def rmsnorm(X16: np.ndarray, gamma16: np.ndarray, eps: float) -> np.ndarray:
    """fp16 bits of the RMS-normalized rows (step 6 of comet_oracle.c)."""
    X = np.ascontiguousarray(X16, dtype=np.uint16)
    g = np.ascontiguousarray(gamma16, dtype=np.uint16)
    M, K = X.shape
    assert g.shape == (K,)
    out = np.empty((M, K), np.uint16)
    _check(lib().orc_rmsnorm_rows(_p(X), M, K, K, _p(g), ctypes.c_float(eps), _p(out), K), "orc_rmsnorm_rows")
    return out


def double_to_half(v: float) -> int:
    return int(lib().orc_double_to_half(ctypes.c_double(v)))


def silu_mul(g16: np.ndarray, u16: np.ndarray) -> np.ndarray:
    """fp16 bits of fp16(silu(g) u), element-wise (step 7 of comet_oracle.c)."""
    g = np.ascontiguousarray(g16, dtype=np.uint16)
    u = np.ascontiguousarray(u16, dtype=np.uint16)
    assert g.shape == u.shape
    h = np.empty_like(g)
    lib().orc_silu_mul_array(_p(g), _p(u), _p(h), g.size)
    return h


def swiglu(G16: np.ndarray, U16: np.ndarray) -> np.ndarray:
    """fp16 bits of the down projection's input rows from the gate and up rows."""
    G = np.ascontiguousarray(G16, dtype=np.uint16)
    U = np.ascontiguousarray(U16, dtype=np.uint16)
    assert G.shape == U.shape and G.ndim == 2
    M, K = G.shape
    H = np.empty((M, K), np.uint16)
    _check(lib().orc_swiglu_rows(_p(G), _p(U), M, K, K, _p(H), K), "orc_swiglu_rows")
    return H


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on."""
    lib().orc_set_threads(int(n))


def quantize_layer(X16, W16, score, nb8):
    """Every logical array of one layer (all rows): a dict."""
    perm, flags = channel_order(score, nb8)
    qw, sw16, wsum = quantize_weights(W16, perm)
    qa, sa = quantize_activations(X16, perm, flags)
    return {"perm": perm, "flags": flags, "qw": qw, "sw16": sw16, "wsum": wsum,
            "qa": qa, "sa": sa}


def quantize_layer_asym(X16, W16, score, nb8):
    """quantize_layer with asymmetric 4-bit activation blocks (step 3b)."""
    perm, flags = channel_order(score, nb8)
    qw, sw16, wsum = quantize_weights(W16, perm)
    qa, u4, sa, za = quantize_activations_asym(X16, perm, flags)
    return {"perm": perm, "flags": flags, "qw": qw, "sw16": sw16, "wsum": wsum,
            "qa": qa, "u4": u4, "sa": sa, "za": za}


def reference(X16, W16, score, nb8, rows=None):
    """Full oracle result for rows (default all): quantized arrays plus P, y32, Y16, yexact."""
    d = quantize_layer(X16, W16, score, nb8)
    M = X16.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    P = block_partials(d["qa"], d["qw"], (m0, m1))
    y32, Y16, ye = epilogue(P, d["sa"][m0:m1], d["sw16"])
    d.update({"P": P, "y32": y32, "Y16": Y16, "yexact": ye, "rows": (m0, m1)})
    return d


# ----------------------------------------------------------------------------
# Step 10: QUIK's FP16 outlier columns
# ----------------------------------------------------------------------------

def quik_split(score: np.ndarray, nb8: int, nf: int):
    """(perm [K], flags [nb'] of the K' = K - nf quantized channels): step 1's
    order over all K; the last nf positions stay fp16, the last nb8 blocks of
    the first K' are 8-bit."""
    K = int(score.shape[0])
    assert nf % 128 == 0 and 0 <= nf < K
    perm, _ = channel_order(score, 0)
    kq = K - nf
    flags = np.zeros(kq // 128, np.uint8)
    if nb8:
        flags[-nb8:] = 1
    return perm, flags


def quik_outlier_add(Xf16, Wf16, y32, yexact):
    """Step 10's merge, in place on copies: (y32, Y16, yexact) with the fp16
    outlier part added to step 5's results."""
    Xf = np.ascontiguousarray(Xf16, dtype=np.uint16)
    Wf = np.ascontiguousarray(Wf16, dtype=np.uint16)
    y = np.array(y32, dtype=np.float32, copy=True)
    ye = np.array(yexact, dtype=np.float64, copy=True)
    rows, N = y.shape
    nf = Xf.shape[1]
    assert Xf.shape == (rows, nf) and Wf.shape == (N, nf)
    Y16 = np.zeros((rows, N), np.uint16)
    _check(lib().orc_quik_outlier_add(_p(Xf), _p(Wf), rows, N, nf, _p(y), _p(Y16), _p(ye)),
           "quik_outlier_add")
    return y, Y16, ye


def quik_layer(X16, W16, score, nb8, nf, rows=None):
    """Every logical array of the QUIK variant and its result for rows
    (default all): the quantized part over perm[:K - nf] (steps 2-5), Xf / Wf
    the fp16 columns perm[K - nf:], and the merged y32, Y16, yexact."""
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    M, K = X16.shape
    perm, flags = quik_split(score, nb8, nf)
    kq = K - nf
    pq = np.ascontiguousarray(perm[:kq])
    pf = perm[kq:]
    qw, sw16, wsum = quantize_weights(np.ascontiguousarray(W16[:, pq]), np.arange(kq, dtype=np.int32))
    qa, sa = quantize_activations(np.ascontiguousarray(X16[:, pq]), np.arange(kq, dtype=np.int32), flags)
    m0, m1 = rows if rows is not None else (0, M)
    P = block_partials(qa, qw, (m0, m1))
    y32, _, ye = epilogue(P, sa[m0:m1], sw16)
    Xf = np.ascontiguousarray(X16[m0:m1][:, pf])
    Wf = np.ascontiguousarray(W16[:, pf])
    y32, Y16, ye = quik_outlier_add(Xf, Wf, y32, ye)
    return {"perm": perm, "flags": flags, "qw": qw, "sw16": sw16, "wsum": wsum, "qa": qa, "sa": sa,
            "Xf_all": np.ascontiguousarray(X16[:, pf]), "Wf": Wf, "P": P, "y32": y32, "Y16": Y16,
            "yexact": ye, "rows": (m0, m1)}


# ----------------------------------------------------------------------------
# Step 8: QoQ progressive group quantization (W4A8)
# ----------------------------------------------------------------------------

def qoq_group(w8: np.ndarray):
    """(s2, z, u) of one group of 8-bit weights."""
    w8 = np.ascontiguousarray(w8, dtype=np.int8)
    u = np.zeros(len(w8), np.uint8)
    z = ctypes.c_int()
    s2 = lib().orc_qoq_group(_p(w8), len(w8), ctypes.byref(z), _p(u))
    return s2, z.value, u


def qoq_quantize_weights(W16: np.ndarray, perm: np.ndarray):
    """(s1 fp16 bits [N], w8 int8 [N, K], s2 uint8 [N, nb], z uint8 [N, nb], u uint8 [N, K])."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    N, K = W16.shape
    nb = K // 128
    s1 = np.zeros(N, np.uint16)
    w8 = np.zeros((N, K), np.int8)
    s2 = np.zeros((N, nb), np.uint8)
    z = np.zeros((N, nb), np.uint8)
    u = np.zeros((N, K), np.uint8)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    _check(lib().orc_qoq_quantize_weights(_p(W16), N, K, _p(perm), _p(s1), _p(w8), _p(s2), _p(z), _p(u)),
           "qoq_quantize_weights")
    return s1, w8, s2, z, u


def qoq_quantize_activations(X16: np.ndarray, perm: np.ndarray):
    """(qa int8 [M, K] permuted, sa float32 [M])."""
    X16 = np.ascontiguousarray(X16, dtype=np.uint16)
    M, K = X16.shape
    qa = np.zeros((M, K), np.int8)
    sa = np.zeros(M, np.float32)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    _check(lib().orc_qoq_quantize_activations(_p(X16), M, K, K, _p(perm), _p(qa), _p(sa)),
           "qoq_quantize_activations")
    return qa, sa


def qoq_gemm(qa, sa, u, s2, z, s1, rows=None):
    """(P int32 [rows, N], y32, Y16, yexact) for rows (default all)."""
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.uint8)
    s2 = np.ascontiguousarray(s2, dtype=np.uint8)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    s1 = np.ascontiguousarray(s1, dtype=np.uint16)
    M, K = qa.shape
    N = u.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    P = np.zeros((m1 - m0, N), np.int32)
    y32 = np.zeros((m1 - m0, N), np.float32)
    Y16 = np.zeros((m1 - m0, N), np.uint16)
    ye = np.zeros((m1 - m0, N), np.float64)
    _check(lib().orc_qoq_gemm(_p(qa), _p(sa), _p(u), _p(s2), _p(z), _p(s1), M, N, K, m0, m1, _p(P), _p(y32),
                              _p(Y16), _p(ye)), "qoq_gemm")
    return P, y32, Y16, ye


def qoq_layer(X16, W16, score, rows=None):
    """Every logical array of a QoQ W4A8 layer plus its product rows."""
    perm, _ = channel_order(score, 0)
    s1, w8, s2, z, u = qoq_quantize_weights(W16, perm)
    qa, sa = qoq_quantize_activations(X16, perm)
    P, y32, Y16, ye = qoq_gemm(qa, sa, u, s2, z, s1, rows)
    return {"perm": perm, "s1": s1, "w8": w8, "s2": s2, "z": z, "u": u, "qa": qa, "sa": sa,
            "P": P, "y32": y32, "Y16": Y16, "yexact": ye}


# ----------------------------------------------------------------------------
# Step 9: KV4 decode attention
# ----------------------------------------------------------------------------

def kv4_quantize(V16: np.ndarray):
    """Codes uint8 [n, d], steps fp16 bits [n], zero points uint8 [n] of n vectors."""
    V16 = np.ascontiguousarray(V16, dtype=np.uint16)
    n, d = V16.shape
    u = np.zeros((n, d), np.uint8)
    s16 = np.zeros(n, np.uint16)
    z = np.zeros(n, np.uint8)
    _check(lib().orc_kv4_quantize(_p(V16), n, d, _p(u), _p(s16), _p(z)), "kv4_quantize")
    return u, s16, z


def kv4_attention(q16, uk, sk, zk, uv, sv, zv):
    """q16 fp16 bits [H, d]; codes [H, T, d]; steps [H, T]; zero points [H, T] ->
    out float64 [H, d]."""
    q16 = np.ascontiguousarray(q16, dtype=np.uint16)
    H, d = q16.shape
    T = uk.shape[1]
    out = np.zeros((H, d), np.float64)
    args = [np.ascontiguousarray(a) for a in (uk, sk, zk, uv, sv, zv)]
    _check(lib().orc_kv4_attention(_p(q16), *[_p(a) for a in args], H, T, d, _p(out)), "kv4_attention")
    return out
