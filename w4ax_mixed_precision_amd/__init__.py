"""Python binding of libcomet_w4ax.so (the W4Ax mixed-precision GEMM for gfx950).

Argument marshalling only: every step of the online path runs in the
library's HIP kernels. PyTorch supplies device memory and the current HIP
stream; numpy carries the host arrays of the offline packing step.

The library must have been built (``__graft_entry__.build()`` or
``python w4ax_mixed_precision_amd/build.py``); importing the binding without
it raises immediately, there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcomet_w4ax.so")

COMET_OK = 0
STATUS_NAMES = {0: "COMET_OK", 1: "COMET_ERR_NULL", 2: "COMET_ERR_SHAPE", 3: "COMET_ERR_ALIGN",
                4: "COMET_ERR_ARG", 5: "COMET_ERR_WORKSPACE", 6: "COMET_ERR_HIP",
                7: "COMET_ERR_UNSUPPORTED"}


class CometError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} -> {STATUS_NAMES.get(status, status)}: "
                         f"{lib().comet_status_string(status).decode()}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library, with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.comet_pack_weights.argtypes = [P, I, I, P, I, P, P, P, P, P]
    L.comet_quant_act.argtypes = [P, I, I, I, P, I, P, P, P]
    L.comet_w4ax_gemm.argtypes = [P, P, P, P, P, I, I, I, I, P, I, P, Z, P]
    L.comet_w4ax_gemm_partials.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P]
    L.comet_w4ax_gemm_workspace_bytes.argtypes = [I, I, I, I]
    L.comet_w4ax_gemm_workspace_bytes.restype = Z
    L.comet_xq_fp6_bytes.argtypes = [I, I, I]
    L.comet_xq_fp6_bytes.restype = Z
    L.comet_wq_fp6_bytes.argtypes = [I, I, I]
    L.comet_wq_fp6_bytes.restype = Z
    L.comet_repack_weights_fp6.argtypes = [P, I, I, I, P]
    L.comet_quant_act_fp6.argtypes = [P, I, I, I, P, I, P, P, P]
    L.comet_w4ax_gemm_fp6.argtypes = [P, P, P, P, I, I, I, I, P, I, P, Z, P]
    L.comet_w4ax_gemm_fp6_partials.argtypes = [P, P, P, P, I, I, I, I, I, I, P, I, P, Z, P]
    L.comet_w4ax_gemm_fp6_noalloc.argtypes = [P, P, P, P, I, I, I, I, P, I, P]
    L.comet_w4ax_gemm_fp6_workspace_bytes.argtypes = [I, I, I, I]
    L.comet_w4ax_gemm_fp6_workspace_bytes.restype = Z
    L.comet_pack_weights_quik.argtypes = [P, I, I, P, I, P, P, P, P, P]
    L.comet_xf_bytes.argtypes = [I, I]
    L.comet_xf_bytes.restype = Z
    L.comet_quant_act_quik_fp6.argtypes = [P, I, I, I, P, I, I, P, P, P, P]
    L.comet_w4ax_gemm_quik_fp6.argtypes = [P, P, P, P, I, P, P, I, I, I, I, P, I, P, Z, P]
    L.comet_quant_act_asym.argtypes = [P, I, I, I, P, I, P, P, P, P]
    L.comet_pack_weights_qoq.argtypes = [P, I, I, P, P, P, P, P]
    L.comet_quant_act_token_i8.argtypes = [P, I, I, I, P, P, P, P]
    L.comet_w4a8_qoq_gemm.argtypes = [P, P, P, P, P, I, I, I, P, I, P]
    L.comet_w4a8_qoq_gemm_products.argtypes = [P, P, P, P, P, I, I, I, P, P]
    L.comet_x_zero_bytes.argtypes = [I, I]
    L.comet_kv4_quantize.argtypes = [P, I, I, I, I, I, I, P, P, P, P]
    L.comet_kv4_attention_workspace_bytes.argtypes = [I, I, I]
    L.comet_kv4_attention_workspace_bytes.restype = Z
    L.comet_kv4_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P, Z, P]
    L.comet_kv4_attention_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, P, I, I, P, P, Z, P]
    L.comet_x_zero_bytes.restype = Z
    L.comet_w4ax_gemm_asym.argtypes = [P, P, P, P, P, P, I, I, I, I, P, I, P, Z, P]
    L.comet_w4ax_gemm_asym_partials.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P]
    F = ctypes.c_float
    L.comet_rmsnorm_quant_act.argtypes = [P, I, I, I, P, F, P, I, P, P, P]
    L.comet_rmsnorm_quant_act_fp6.argtypes = [P, I, I, I, P, F, P, I, P, P, P]
    L.comet_rmsnorm.argtypes = [P, I, I, I, P, F, P, I, P]
    L.comet_permute_channels.argtypes = [P, P, I, P]
    L.comet_swiglu_quant_act.argtypes = [P, P, I, I, I, P, I, P, P, P]
    L.comet_swiglu_quant_act_fp6.argtypes = [P, P, I, I, I, P, I, P, P, P]
    L.comet_swiglu.argtypes = [P, P, I, I, I, P, I, P]
    L.comet_status_string.argtypes = [I]
    L.comet_status_string.restype = ctypes.c_char_p
    L.comet_version.restype = ctypes.c_char_p
    for f in ("comet_pack_weights", "comet_quant_act", "comet_w4ax_gemm",
              "comet_w4ax_gemm_partials", "comet_repack_weights_fp6", "comet_quant_act_fp6",
              "comet_w4ax_gemm_fp6", "comet_w4ax_gemm_fp6_partials", "comet_w4ax_gemm_fp6_workspace_bytes",
              "comet_w4ax_gemm_fp6_noalloc", "comet_rmsnorm_quant_act",
              "comet_rmsnorm_quant_act_fp6", "comet_rmsnorm", "comet_permute_channels",
              "comet_swiglu_quant_act", "comet_swiglu_quant_act_fp6", "comet_swiglu",
              "comet_quant_act_asym", "comet_w4ax_gemm_asym", "comet_w4ax_gemm_asym_partials",
              "comet_pack_weights_qoq", "comet_quant_act_token_i8", "comet_w4a8_qoq_gemm",
              "comet_w4a8_qoq_gemm_products", "comet_kv4_quantize", "comet_kv4_attention",
              "comet_kv4_attention_varlen", "comet_pack_weights_quik", "comet_quant_act_quik_fp6", "comet_w4ax_gemm_quik_fp6"):
        getattr(L, f).restype = I
    _lib = L
    return L


EXPORTS = ("comet_pack_weights", "comet_quant_act", "comet_w4ax_gemm",
           "comet_w4ax_gemm_workspace_bytes", "comet_w4ax_gemm_partials",
           "comet_xq_fp6_bytes", "comet_wq_fp6_bytes", "comet_repack_weights_fp6",
           "comet_quant_act_fp6", "comet_w4ax_gemm_fp6", "comet_w4ax_gemm_fp6_partials",
           "comet_w4ax_gemm_fp6_workspace_bytes", "comet_w4ax_gemm_fp6_noalloc",
           "comet_rmsnorm_quant_act", "comet_rmsnorm_quant_act_fp6", "comet_rmsnorm",
           "comet_permute_channels", "comet_swiglu_quant_act", "comet_swiglu_quant_act_fp6", "comet_swiglu",
           "comet_quant_act_asym", "comet_x_zero_bytes", "comet_w4ax_gemm_asym",
           "comet_w4ax_gemm_asym_partials", "comet_pack_weights_qoq", "comet_quant_act_token_i8",
           "comet_w4a8_qoq_gemm", "comet_w4a8_qoq_gemm_products", "comet_kv4_quantize",
           "comet_kv4_attention_workspace_bytes", "comet_kv4_attention", "comet_kv4_attention_varlen",
           "comet_pack_weights_quik",
           "comet_xf_bytes", "comet_quant_act_quik_fp6", "comet_w4ax_gemm_quik_fp6", "comet_status_string",
           "comet_version")


def _check(call: str, rc: int):
    if rc != COMET_OK:
        raise CometError(call, rc)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def nblocks(K: int) -> int:
    return K // 128


def xq_bytes(M: int, K: int, nb8: int) -> int:
    nb = K // 128
    return M * (64 * (nb - nb8) + 128 * nb8)


def xq_fp6_bytes(M: int, K: int, nb8: int) -> int:
    nb = K // 128
    mp = (M + 15) // 16 * 16          # rows padded to whole 16-row tiles
    return mp * (96 * (nb - nb8) + 128 * nb8)


def wq_fp6_bytes(N: int, K: int, nb8: int) -> int:
    nb = K // 128
    return N * (96 * (nb - nb8) + 64 * nb8)


# ----------------------------------------------------------------------------
# Offline (host)
# ----------------------------------------------------------------------------

def comet_pack_weights(W16: np.ndarray, score: np.ndarray, nb8: int) -> dict:
    """Rank channels, quantize and pack W. Host numpy in, host numpy out:
    perm int32 [K], flags uint8 [nb], Wq uint8 [N*K/2], w_scale uint16 [nb, N],
    w_sum int16 [nb, N]."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    score = np.ascontiguousarray(score, dtype=np.float32)
    N, K = W16.shape
    if score.shape != (K,):
        raise ValueError("score must have K entries")
    nb = max(K // 128, 1)
    out = {"perm": np.zeros(K, np.int32), "flags": np.zeros(nb, np.uint8),
           "Wq": np.zeros(N * K // 2, np.uint8), "w_scale": np.zeros((nb, N), np.uint16),
           "w_sum": np.zeros((nb, N), np.int16)}
    rc = lib().comet_pack_weights(_np_ptr(W16), N, K, _np_ptr(score), int(nb8),
                                  _np_ptr(out["perm"]), _np_ptr(out["flags"]), _np_ptr(out["Wq"]),
                                  _np_ptr(out["w_scale"]), _np_ptr(out["w_sum"]))
    _check("comet_pack_weights", rc)
    out["N"], out["K"], out["nb8"] = N, K, int(nb8)
    return out


def comet_repack_weights_fp6(packed: dict) -> dict:
    """Add the FP6-layout weights (key "WqF") to a bundle from comet_pack_weights."""
    N, K, nb8 = packed["N"], packed["K"], packed["nb8"]
    WqF = np.zeros(wq_fp6_bytes(N, K, nb8), np.uint8)
    rc = lib().comet_repack_weights_fp6(_np_ptr(np.ascontiguousarray(packed["Wq"])), N, K, int(nb8),
                                        _np_ptr(WqF))
    _check("comet_repack_weights_fp6", rc)
    packed["WqF"] = WqF
    return packed


def upload_weights(packed: dict, device="cuda") -> dict:
    """Copy the packed weight bundle to device tensors (torch only as memory)."""
    import torch
    d = {"perm": torch.from_numpy(packed["perm"]).to(device),
         "w_scale": torch.from_numpy(packed["w_scale"].view(np.int16)).to(device),
         "w_sum": torch.from_numpy(packed["w_sum"]).to(device)}
    if "Wq" in packed:
        d["Wq"] = torch.from_numpy(packed["Wq"]).to(device)
    if "WqF" in packed:
        d["WqF"] = torch.from_numpy(packed["WqF"]).to(device)
    if packed.get("nf", 0) > 0:
        d["Wf"] = torch.from_numpy(packed["Wf"].view(np.int16)).to(device)
    d.update({k: packed[k] for k in ("N", "K", "nb8")})
    d["nf"] = packed.get("nf", 0)
    return d


def comet_pack_weights_quik(W16: np.ndarray, score: np.ndarray, nb8: int, nf: int) -> dict:
    """QUIK's split (host): perm int32 [K]; the quantized pack of the first
    K - nf permuted channels (Wq, w_scale, w_sum, and its FP6 repack WqF with
    nb8 8-bit blocks); Wf uint16 [N * nf], the fp16 outlier fragments."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    score = np.ascontiguousarray(score, dtype=np.float32)
    N, K = W16.shape
    if score.shape != (K,):
        raise ValueError("score must have K entries")
    kq = K - int(nf)
    nbq = max(kq // 128, 1)
    out = {"perm": np.zeros(K, np.int32), "Wq": np.zeros(N * max(kq, 0) // 2, np.uint8),
           "w_scale": np.zeros((nbq, N), np.uint16), "w_sum": np.zeros((nbq, N), np.int16),
           "Wf": np.zeros(max(N * int(nf), 1), np.uint16)}
    rc = lib().comet_pack_weights_quik(_np_ptr(W16), N, K, _np_ptr(score), int(nf), _np_ptr(out["perm"]),
                                       _np_ptr(out["Wq"]), _np_ptr(out["w_scale"]), _np_ptr(out["w_sum"]),
                                       _np_ptr(out["Wf"]))
    _check("comet_pack_weights_quik", rc)
    WqF = np.zeros(wq_fp6_bytes(N, kq, nb8), np.uint8)
    _check("comet_repack_weights_fp6",
           lib().comet_repack_weights_fp6(_np_ptr(out["Wq"]), N, kq, int(nb8), _np_ptr(WqF)))
    out.update({"WqF": WqF, "N": N, "K": kq, "K_full": K, "nb8": int(nb8), "nf": int(nf)})
    return out


# ----------------------------------------------------------------------------
# Online (device)
# ----------------------------------------------------------------------------

def comet_quant_act(X, perm, nb8: int, Xq=None, x_scale=None, stream=None):
    """X: fp16 cuda tensor [M, ldx] (uses the first K = len(perm) columns).
    Returns (Xq uint8 [xq_bytes], x_scale float32 [nb, M])."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    if Xq is None:
        Xq = torch.empty(xq_bytes(M, K, nb8), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty((K // 128, M), dtype=torch.float32, device=X.device)
    rc = lib().comet_quant_act(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(perm), int(nb8),
                               _dev_ptr(Xq), _dev_ptr(x_scale), _stream(stream))
    _check("comet_quant_act", rc)
    return Xq, x_scale


def x_zero_bytes(M: int, K: int) -> int:
    return int(lib().comet_x_zero_bytes(M, K))


def comet_quant_act_asym(X, perm, nb8: int, Xq=None, x_scale=None, x_zero=None, stream=None):
    """Asymmetric 4-bit blocks: returns (Xq uint8 [xq_bytes], x_scale float32 [nb, M],
    x_zero uint8 [nb, Mp], Mp = M rounded up to 16)."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    if Xq is None:
        Xq = torch.empty(xq_bytes(M, K, nb8), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty((K // 128, M), dtype=torch.float32, device=X.device)
    if x_zero is None:
        x_zero = torch.zeros((K // 128, (M + 15) // 16 * 16), dtype=torch.uint8, device=X.device)
    rc = lib().comet_quant_act_asym(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(perm), int(nb8),
                                    _dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(x_zero), _stream(stream))
    _check("comet_quant_act_asym", rc)
    return Xq, x_scale, x_zero


def comet_w4ax_gemm_asym(Xq, x_scale, x_zero, w: dict, M: int, Y=None, stream=None):
    """Y fp16 [M, N] from asymmetric activation codes (comet_quant_act_asym)."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    rc = lib().comet_w4ax_gemm_asym(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(x_zero), _dev_ptr(w["Wq"]),
                                    _dev_ptr(w["w_scale"]), _dev_ptr(w["w_sum"]), int(nb8), M, N, K,
                                    _dev_ptr(Y), Y.stride(0), None, 0, _stream(stream))
    _check("comet_w4ax_gemm_asym", rc)
    return Y


def comet_w4ax_gemm_asym_partials(Xq, x_scale, x_zero, w: dict, M: int, m_begin: int = 0,
                                  m_count: int | None = None, P=None, stream=None):
    """Exact INT32 block partials (asymmetric codes) of rows [m_begin, m_begin + m_count)."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    m_count = M - m_begin if m_count is None else m_count
    if P is None:
        P = torch.empty((m_count, N, K // 128), dtype=torch.int32, device=Xq.device)
    rc = lib().comet_w4ax_gemm_asym_partials(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(x_zero),
                                             _dev_ptr(w["Wq"]), _dev_ptr(w["w_scale"]), _dev_ptr(w["w_sum"]),
                                             int(nb8), M, N, K, m_begin, m_count, _dev_ptr(P), _stream(stream))
    _check("comet_w4ax_gemm_asym_partials", rc)
    return P


def comet_pack_weights_qoq(W16: np.ndarray, score: np.ndarray) -> dict:
    """QoQ progressive group quantization of W (host): perm, Wu (unsigned codes,
    fragment order), s1 fp16 bits [N], s2z uint16 [nb, N] (s2 | z << 8)."""
    W16 = np.ascontiguousarray(W16, dtype=np.uint16)
    N, K = W16.shape
    score = np.ascontiguousarray(score, dtype=np.float32)
    perm = np.zeros(K, np.int32)
    Wu = np.zeros(N * K // 2, np.uint8)
    s1 = np.zeros(N, np.uint16)
    s2z = np.zeros((K // 128, N), np.uint16)
    _check("comet_pack_weights_qoq", lib().comet_pack_weights_qoq(_np_ptr(W16), N, K, _np_ptr(score),
                                                                  _np_ptr(perm), _np_ptr(Wu), _np_ptr(s1),
                                                                  _np_ptr(s2z)))
    return {"perm": perm, "Wu": Wu, "s1": s1, "s2z": s2z, "N": N, "K": K}


def upload_qoq(pk: dict, device="cuda") -> dict:
    import torch
    d = {k: torch.from_numpy(pk[k].view(np.int16) if pk[k].dtype == np.uint16 else pk[k]).to(device)
         for k in ("perm", "Wu", "s1", "s2z")}
    d.update({"N": pk["N"], "K": pk["K"]})
    return d


def comet_quant_act_token_i8(X, perm, Xq=None, x_scale=None, stream=None):
    """Per-token INT8 codes (8-bit slabs, M*K bytes) and x_scale float32 [M]."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    if Xq is None:
        Xq = torch.empty(M * K, dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    rc = lib().comet_quant_act_token_i8(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(perm), _dev_ptr(Xq),
                                        _dev_ptr(x_scale), _stream(stream))
    _check("comet_quant_act_token_i8", rc)
    return Xq, x_scale


def comet_w4a8_qoq_gemm(Xq, x_scale, w: dict, M: int, Y=None, stream=None):
    import torch
    N, K = w["N"], w["K"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    rc = lib().comet_w4a8_qoq_gemm(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["Wu"]), _dev_ptr(w["s2z"]),
                                   _dev_ptr(w["s1"]), M, N, K, _dev_ptr(Y), Y.stride(0), _stream(stream))
    _check("comet_w4a8_qoq_gemm", rc)
    return Y


def comet_w4a8_qoq_gemm_products(Xq, x_scale, w: dict, M: int, P=None, stream=None):
    import torch
    N, K = w["N"], w["K"]
    if P is None:
        P = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    rc = lib().comet_w4a8_qoq_gemm_products(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["Wu"]),
                                            _dev_ptr(w["s2z"]), _dev_ptr(w["s1"]), M, N, K, _dev_ptr(P),
                                            _stream(stream))
    _check("comet_w4a8_qoq_gemm_products", rc)
    return P


def kv4_cache(H: int, tcap: int, d: int, device="cuda") -> dict:
    """An empty KV4 cache of H heads and tcap slots (codes, step, zero)."""
    import torch
    return {"codes": torch.zeros(H * tcap * d // 2, dtype=torch.uint8, device=device),
            "step": torch.zeros(H * tcap, dtype=torch.int16, device=device),
            "zero": torch.zeros(H * tcap, dtype=torch.uint8, device=device),
            "H": H, "tcap": tcap, "d": d}


def comet_kv4_quantize(X, cache: dict, pos: int, stream=None):
    """Quantize X fp16 [ntok, >= H d] (token rows, heads side by side) into
    cache slots pos .. pos + ntok - 1 of every head."""
    ntok = X.shape[0]
    rc = lib().comet_kv4_quantize(_dev_ptr(X), ntok, cache["H"], cache["d"], X.stride(0), pos, cache["tcap"],
                                  _dev_ptr(cache["codes"]), _dev_ptr(cache["step"]), _dev_ptr(cache["zero"]),
                                  _stream(stream))
    _check("comet_kv4_quantize", rc)


def comet_kv4_attention(q, kcache: dict, vcache: dict, T: int, group: int = 1, out=None, workspace=None,
                        stream=None):
    """Decode attention of q fp16 [Hq, d] over the first T slots of the caches."""
    import torch
    Hq, d = q.shape
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float16, device=q.device)
    nbytes = lib().comet_kv4_attention_workspace_bytes(Hq, d, T)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = lib().comet_kv4_attention(_dev_ptr(q), _dev_ptr(kcache["codes"]), _dev_ptr(kcache["step"]),
                                   _dev_ptr(kcache["zero"]), _dev_ptr(vcache["codes"]), _dev_ptr(vcache["step"]),
                                   _dev_ptr(vcache["zero"]), Hq, group, d, T, kcache["tcap"], _dev_ptr(out),
                                   _dev_ptr(workspace), workspace.numel(), _stream(stream))
    _check("comet_kv4_attention", rc)
    return out


def comet_kv4_attention_varlen(q, kcache: dict, vcache: dict, T_kv, T_max: int, group: int = 1, out=None,
                               workspace=None, stream=None):
    """Decode attention of q fp16 [Hq, d]; kv head g over its first T_kv[g]
    slots (T_kv: int32 cuda tensor [Hq / group], values clamped to [0, T_max])."""
    import torch
    Hq, d = q.shape
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float16, device=q.device)
    nbytes = lib().comet_kv4_attention_workspace_bytes(Hq, d, T_max)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = lib().comet_kv4_attention_varlen(_dev_ptr(q), _dev_ptr(kcache["codes"]), _dev_ptr(kcache["step"]),
                                          _dev_ptr(kcache["zero"]), _dev_ptr(vcache["codes"]),
                                          _dev_ptr(vcache["step"]), _dev_ptr(vcache["zero"]), Hq, group, d,
                                          _dev_ptr(T_kv), T_max, kcache["tcap"], _dev_ptr(out), _dev_ptr(workspace),
                                          workspace.numel(), _stream(stream))
    _check("comet_kv4_attention_varlen", rc)
    return out


def comet_permute_channels(v: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Host: out[k] = v[perm[k]] (fp16 bits), e.g. the RMSNorm weight into the permuted order."""
    v = np.ascontiguousarray(v, dtype=np.uint16)
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    out = np.empty(perm.shape[0], np.uint16)
    _check("comet_permute_channels", lib().comet_permute_channels(
        v.ctypes.data_as(ctypes.c_void_p), perm.ctypes.data_as(ctypes.c_void_p), perm.shape[0],
        out.ctypes.data_as(ctypes.c_void_p)))
    return out


def comet_rmsnorm_quant_act(X, gamma_perm, eps: float, perm, nb8: int, Xq=None, x_scale=None, fp6=False,
                            stream=None):
    """RMS normalization fused into the quantizer (either layout). X: fp16 cuda tensor [M, ldx] of
    un-normalized rows; gamma_perm: fp16 cuda tensor [K] in permuted order."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    if Xq is None:
        n = xq_fp6_bytes(M, K, nb8) if fp6 else xq_bytes(M, K, nb8)
        Xq = torch.empty(n, dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty((K // 128, M), dtype=torch.float32, device=X.device)
    call = "comet_rmsnorm_quant_act_fp6" if fp6 else "comet_rmsnorm_quant_act"
    rc = getattr(lib(), call)(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(gamma_perm), float(eps), _dev_ptr(perm),
                              int(nb8), _dev_ptr(Xq), _dev_ptr(x_scale), _stream(stream))
    _check(call, rc)
    return Xq, x_scale


def comet_rmsnorm(X, gamma, eps: float, K: int | None = None, Xn=None, stream=None):
    """The normalization on its own: fp16 [M, K] in the original channel order."""
    import torch
    M, ldx = X.shape
    K = ldx if K is None else K
    if Xn is None:
        Xn = torch.empty((M, K), dtype=torch.float16, device=X.device)
    rc = lib().comet_rmsnorm(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(gamma), float(eps), _dev_ptr(Xn),
                             Xn.stride(0), _stream(stream))
    _check("comet_rmsnorm", rc)
    return Xn


def comet_swiglu_quant_act(gate, up, perm, nb8: int, Xq=None, x_scale=None, fp6=False, stream=None):
    """SwiGLU fused into the quantizer (either layout). gate, up: fp16 cuda tensors [M, K] (views
    with one common row stride, e.g. the two halves of a [M, 2K] projection output)."""
    import torch
    M = gate.shape[0]
    K = perm.shape[0]
    if tuple(up.shape) != tuple(gate.shape) or up.stride(0) != gate.stride(0):
        raise ValueError("gate and up must have the same shape and row stride")
    if Xq is None:
        n = xq_fp6_bytes(M, K, nb8) if fp6 else xq_bytes(M, K, nb8)
        Xq = torch.empty(n, dtype=torch.uint8, device=gate.device)
    if x_scale is None:
        x_scale = torch.empty((K // 128, M), dtype=torch.float32, device=gate.device)
    call = "comet_swiglu_quant_act_fp6" if fp6 else "comet_swiglu_quant_act"
    rc = getattr(lib(), call)(_dev_ptr(gate), _dev_ptr(up), M, K, gate.stride(0), _dev_ptr(perm), int(nb8),
                              _dev_ptr(Xq), _dev_ptr(x_scale), _stream(stream))
    _check(call, rc)
    return Xq, x_scale


def comet_swiglu(gate, up, K: int | None = None, H=None, stream=None):
    """The SwiGLU on its own: fp16 [M, K] = fp16(silu(gate) up), original channel order."""
    import torch
    M, ld = gate.shape
    K = ld if K is None else K
    if up.stride(0) != gate.stride(0):
        raise ValueError("gate and up must share their row stride")
    if H is None:
        H = torch.empty((M, K), dtype=torch.float16, device=gate.device)
    rc = lib().comet_swiglu(_dev_ptr(gate), _dev_ptr(up), M, K, gate.stride(0), _dev_ptr(H), H.stride(0),
                            _stream(stream))
    _check("comet_swiglu", rc)
    return H


def workspace_bytes(M: int, N: int, K: int, nb8: int) -> int:
    return int(lib().comet_w4ax_gemm_workspace_bytes(M, N, K, nb8))


def comet_w4ax_gemm(Xq, x_scale, w: dict, M: int, Y=None, workspace=None, stream=None):
    """Y fp16 [M, N] = dequant(Xq) dequant(Wq)^T for the uploaded weight bundle `w`."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    need = workspace_bytes(M, N, K, nb8)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    ws_ptr = _dev_ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    rc = lib().comet_w4ax_gemm(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["Wq"]),
                               _dev_ptr(w["w_scale"]), _dev_ptr(w["w_sum"]), int(nb8), M, N, K,
                               _dev_ptr(Y), Y.stride(0), ws_ptr, ws_bytes, _stream(stream))
    _check("comet_w4ax_gemm", rc)
    return Y


def comet_w4ax_gemm_partials(Xq, x_scale, w: dict, M: int, m_begin: int = 0,
                             m_count: int | None = None, P=None, stream=None):
    """Exact INT32 block partials of rows [m_begin, m_begin + m_count): [m_count, N, nb]."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    m_count = M - m_begin if m_count is None else m_count
    if P is None:
        P = torch.empty((m_count, N, K // 128), dtype=torch.int32, device=Xq.device)
    rc = lib().comet_w4ax_gemm_partials(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["Wq"]),
                                        _dev_ptr(w["w_scale"]), _dev_ptr(w["w_sum"]), int(nb8),
                                        M, N, K, m_begin, m_count, _dev_ptr(P), _stream(stream))
    _check("comet_w4ax_gemm_partials", rc)
    return P


def comet_quant_act_fp6(X, perm, nb8: int, Xq=None, x_scale=None, stream=None):
    """comet_quant_act with FP6 codes for the 4-bit blocks.
    Returns (Xq uint8 [xq_fp6_bytes], x_scale float32 [nb, M])."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    if Xq is None:
        Xq = torch.empty(xq_fp6_bytes(M, K, nb8), dtype=torch.uint8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty((K // 128, M), dtype=torch.float32, device=X.device)
    rc = lib().comet_quant_act_fp6(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(perm), int(nb8),
                                   _dev_ptr(Xq), _dev_ptr(x_scale), _stream(stream))
    _check("comet_quant_act_fp6", rc)
    return Xq, x_scale


def fp6_workspace_bytes(M: int, N: int, K: int, nb8: int) -> int:
    return int(lib().comet_w4ax_gemm_fp6_workspace_bytes(M, N, K, int(nb8)))


_WS_CACHE: dict = {}


def fp6_workspace(M: int, N: int, K: int, nb8: int, device):
    """A zeroed device workspace for comet_w4ax_gemm_fp6 of this shape (None if
    the shape needs none), kept per device and reused: the library returns it
    to zero at the end of every call, so calls ordered on one stream can share
    it (calls that may overlap need workspaces of their own)."""
    import torch
    need = fp6_workspace_bytes(M, N, K, nb8)
    if need == 0:
        return None
    dev = torch.device(device)
    key = (dev.type, dev.index if dev.index is not None else torch.cuda.current_device())
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        _WS_CACHE[key] = ws
    return ws


def comet_w4ax_gemm_fp6(Xq, x_scale, w: dict, M: int, Y=None, workspace=None, stream=None):
    """Y fp16 [M, N] from FP6-layout activations and the bundle's FP6 weights.
    `workspace`: a zeroed uint8 device tensor of at least fp6_workspace_bytes()
    (by default a shared one from fp6_workspace())."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    if workspace is None:
        workspace = fp6_workspace(M, N, K, nb8, Xq.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().comet_w4ax_gemm_fp6(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["WqF"]),
                                   _dev_ptr(w["w_scale"]), int(nb8), M, N, K, _dev_ptr(Y), Y.stride(0),
                                   None if workspace is None else _dev_ptr(workspace), wsz, _stream(stream))
    _check("comet_w4ax_gemm_fp6", rc)
    return Y


def xf_bytes(M: int, nf: int) -> int:
    return int(lib().comet_xf_bytes(M, int(nf)))


def comet_quant_act_quik_fp6(X, perm, nb8: int, nf: int, stream=None):
    """QUIK's split of the activations: the FP6-layout codes of the channels
    perm[:K - nf] and the fp16 outlier tiles of perm[K - nf:].
    Returns (Xq, x_scale float32 [(K - nf) / 128, M], Xf int16 tiles)."""
    import torch
    M, ldx = X.shape
    K = perm.shape[0]
    kq = K - int(nf)
    Xq = torch.empty(xq_fp6_bytes(M, kq, nb8), dtype=torch.uint8, device=X.device)
    x_scale = torch.empty((kq // 128, M), dtype=torch.float32, device=X.device)
    Xf = torch.empty(max(xf_bytes(M, nf) // 2, 8), dtype=torch.int16, device=X.device)
    rc = lib().comet_quant_act_quik_fp6(_dev_ptr(X), M, K, X.stride(0), _dev_ptr(perm), int(nb8), int(nf),
                                        _dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(Xf), _stream(stream))
    _check("comet_quant_act_quik_fp6", rc)
    return Xq, x_scale, Xf


def comet_w4ax_gemm_quik_fp6(Xq, x_scale, Xf, w: dict, M: int, Y=None, workspace=None, stream=None):
    """Y fp16 [M, N] of QUIK's split from comet_quant_act_quik_fp6's outputs and
    an uploaded comet_pack_weights_quik bundle (w["K"] = K - nf)."""
    import torch
    N, kq, nb8, nf = w["N"], w["K"], w["nb8"], w["nf"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    if workspace is None:
        workspace = fp6_workspace(M, N, kq, nb8, Xq.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().comet_w4ax_gemm_quik_fp6(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["WqF"]),
                                        _dev_ptr(w["w_scale"]), int(nb8), _dev_ptr(Xf),
                                        _dev_ptr(w["Wf"]) if nf else None, int(nf), M, N, kq + int(nf),
                                        _dev_ptr(Y), Y.stride(0),
                                        None if workspace is None else _dev_ptr(workspace), wsz,
                                        _stream(stream))
    _check("comet_w4ax_gemm_quik_fp6", rc)
    return Y


NOALLOC_SCRATCH_BYTES = 36 << 20      # COMET_NOALLOC_SCRATCH_BYTES of the header


def comet_w4ax_gemm_fp6_noalloc(Xq, x_scale, w: dict, M: int, Y=None, stream=None):
    """comet_w4ax_gemm_fp6 on the library's fixed per-GPU scratch (no workspace
    argument; the call itself allocates nothing)."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    rc = lib().comet_w4ax_gemm_fp6_noalloc(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["WqF"]),
                                           _dev_ptr(w["w_scale"]), int(nb8), M, N, K, _dev_ptr(Y), Y.stride(0),
                                           _stream(stream))
    _check("comet_w4ax_gemm_fp6_noalloc", rc)
    return Y


def comet_w4ax_gemm_fp6_partials(Xq, x_scale, w: dict, M: int, m_begin: int = 0,
                                 m_count: int | None = None, P=None, workspace=None, stream=None,
                                 max_workgroups: int = 0):
    """Exact block partials of the FP6-layout GEMM, [m_count, N, nb] int32."""
    import torch
    N, K, nb8 = w["N"], w["K"], w["nb8"]
    m_count = M - m_begin if m_count is None else m_count
    if P is None:
        P = torch.empty((m_count, N, K // 128), dtype=torch.int32, device=Xq.device)
    if workspace is None:
        workspace = fp6_workspace(M, N, K, nb8, Xq.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().comet_w4ax_gemm_fp6_partials(_dev_ptr(Xq), _dev_ptr(x_scale), _dev_ptr(w["WqF"]),
                                            _dev_ptr(w["w_scale"]), int(nb8), M, N, K, m_begin,
                                            m_count, _dev_ptr(P), int(max_workgroups),
                                            None if workspace is None else _dev_ptr(workspace), wsz,
                                            _stream(stream))
    _check("comet_w4ax_gemm_fp6_partials", rc)
    return P


def version() -> str:
    return lib().comet_version().decode()
