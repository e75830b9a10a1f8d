"""Decoders of the library's packed layouts, written from the layout section of
include/comet_w4ax.h. Tests use them to turn GPU and packer outputs back into
the logical arrays the oracle produces."""
import numpy as np


def _sext4(v):
    v = v.astype(np.int8)
    return np.where(v >= 8, v - 16, v).astype(np.int8)


def decode_wq(Wq: np.ndarray, N: int, K: int) -> np.ndarray:
    """Wq bytes -> q_w int8 [N, K] in permuted channel order."""
    nb = K // 128
    f = np.asarray(Wq, dtype=np.uint8).reshape(N // 16, nb, 4, 16, 16)   # [c, b, g, n16, j]
    lo = _sext4(f & 0xF)
    hi = _sext4(f >> 4)
    q = np.empty((N // 16, 16, nb, 4, 2, 16), np.int8)                   # [c, n16, b, g, half, j]
    q[:, :, :, :, 0, :] = lo.transpose(0, 3, 1, 2, 4)
    q[:, :, :, :, 1, :] = hi.transpose(0, 3, 1, 2, 4)
    return q.reshape(N, K)


def decode_xq(Xq: np.ndarray, M: int, K: int, nb8: int) -> np.ndarray:
    """Xq bytes -> q_a int8 [M, K] in permuted channel order."""
    nb = K // 128
    nb4 = nb - nb8
    Xq = np.asarray(Xq, dtype=np.uint8)
    q = np.empty((M, K), np.int8)
    s4 = Xq[: nb4 * M * 64].reshape(nb4, M, 4, 16)                        # [b, m, g, j]
    lo = (s4 & 0xF).astype(np.int16) - 8
    hi = (s4 >> 4).astype(np.int16) - 8
    blk = np.stack([lo, hi], axis=3).reshape(nb4, M, 128)                 # [b, m, 32g + 16h + j]
    q[:, : nb4 * 128] = blk.transpose(1, 0, 2).reshape(M, nb4 * 128)
    s8 = Xq[nb4 * M * 64:].view(np.int8).reshape(nb8, M, 128)
    q[:, nb4 * 128:] = s8.transpose(1, 0, 2).reshape(M, nb8 * 128)
    return q


def zero_extended_codes_valid(Xq: np.ndarray, M: int, K: int, nb8: int) -> bool:
    """Every 4-bit code of the zero-extended encoding lies in [1, 15]."""
    nb4 = K // 128 - nb8
    s4 = np.asarray(Xq, dtype=np.uint8)[: nb4 * M * 64]
    return bool(np.all((s4 & 0xF) >= 1) and np.all((s4 >> 4) >= 1))
