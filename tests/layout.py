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


def decode_wu(Wu: np.ndarray, N: int, K: int) -> np.ndarray:
    """QoQ pack: unsigned codes u uint8 [N, K] in permuted channel order (the
    fragment order of decode_wq, nibbles read without sign)."""
    nb = K // 128
    f = np.asarray(Wu, dtype=np.uint8).reshape(N // 16, nb, 4, 16, 16)   # [c, b, g, n16, j]
    u = np.empty((N // 16, 16, nb, 4, 2, 16), np.uint8)                  # [c, n16, b, g, half, j]
    u[:, :, :, :, 0, :] = (f & 0xF).transpose(0, 3, 1, 2, 4)
    u[:, :, :, :, 1, :] = (f >> 4).transpose(0, 3, 1, 2, 4)
    return u.reshape(N, K)


def decode_xq_token_i8(Xq: np.ndarray, M: int, K: int) -> np.ndarray:
    """Per-token INT8 slabs ([nb][M][128]) -> q int8 [M, K] in permuted order."""
    nb = K // 128
    s = np.asarray(Xq, dtype=np.uint8).view(np.int8).reshape(nb, M, 128)
    return s.transpose(1, 0, 2).reshape(M, K)


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


def e2m3_value(code: np.ndarray) -> np.ndarray:
    """Value of FP6 E2M3 codes from the format's definition: bit 5 sign, bits
    4..3 exponent (bias 1), bits 2..0 mantissa; exponent 0 is subnormal."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c >> 5 & 1, -1.0, 1.0)
    e = c >> 3 & 3
    m = c & 7
    return s * np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * 2.0 ** (e - 1))


def _codes_from_groups(groups: np.ndarray) -> np.ndarray:
    """[..., 24] bytes of a group string -> [..., 32] 6-bit codes (code j at bits 6j)."""
    bits = np.unpackbits(np.asarray(groups, dtype=np.uint8), axis=-1, bitorder="little")
    bits = bits.reshape(bits.shape[:-1] + (32, 6)).astype(np.int64)
    return (bits << np.arange(6)).sum(-1)


def _fp6_ints(codes: np.ndarray) -> np.ndarray:
    v = e2m3_value(codes)
    assert np.all(v == np.round(v)) and np.all(np.abs(v) <= 7), "FP6 code is not a 4-bit integer"
    assert not np.any(codes == 32), "negative zero code"
    return v.astype(np.int8)


def _tile_rows_index():
    """Byte offsets in a 16-row activation tile of the FP6 layout: row r's
    16-byte piece of group g at 64 r + 16 (g ^ h(r)), its 8-byte tail at
    1024 + 32 r + 8 (g ^ t(r)), h(r) = (r >> 1) & 3,
    t(r) = (r >> 2) & 3. Returns head [16, 4, 16] and tail [16, 4, 8] indices."""
    r = np.arange(16)[:, None]
    g = np.arange(4)[None, :]
    h = (r >> 1) & 3
    t = (r >> 2) & 3
    head = (64 * r + 16 * (g ^ h))[:, :, None] + np.arange(16)
    tail = (1024 + 32 * r + 8 * (g ^ t))[:, :, None] + np.arange(8)
    return head, tail


def decode_xq_fp6(Xq: np.ndarray, M: int, K: int, nb8: int) -> np.ndarray:
    """Xq_fp6 bytes (16-row tiles, rows padded to Mp) -> q_a int8 [M, K] in
    permuted channel order."""
    nb = K // 128
    nb4 = nb - nb8
    Mp = (M + 15) // 16 * 16
    T = Mp // 16
    Xq = np.asarray(Xq, dtype=np.uint8)
    assert Xq.size == Mp * (96 * nb4 + 128 * nb8)
    head, tail = _tile_rows_index()
    q = np.empty((M, K), np.int8)
    tiles = Xq[: nb4 * Mp * 96].reshape(nb4, T, 1536)
    groups = np.concatenate([tiles[:, :, head], tiles[:, :, tail]], axis=-1)      # [b, t, r, g, 24]
    codes = _codes_from_groups(groups).reshape(nb4, Mp, 128)[:, :M]               # padding rows dropped
    vals = _fp6_ints(codes)                                                        # [b, m, 32g + j]
    q[:, : nb4 * 128] = vals.transpose(1, 0, 2).reshape(M, nb4 * 128)
    t8 = Xq[nb4 * Mp * 96:].view(np.int8).reshape(nb8, T, 2, 1024)                 # [b, t, half, byte]
    v8 = t8[:, :, :, head]                                                         # [b, t, h, r, g, j]
    v8 = v8.transpose(0, 1, 3, 4, 2, 5).reshape(nb8, Mp, 128)[:, :M]               # [b, m, 32g + 16h + j]
    q[:, nb4 * 128:] = v8.transpose(1, 0, 2).reshape(M, nb8 * 128)
    return q


def decode_wq_fp6(WqF: np.ndarray, N: int, K: int, nb8: int) -> np.ndarray:
    """Wq_fp6 bytes -> q_w int8 [N, K] in permuted channel order."""
    nb = K // 128
    nb4 = nb - nb8
    G = N // 16
    WqF = np.asarray(WqF, dtype=np.uint8)
    q = np.empty((N, K), np.int8)
    f = WqF[: nb4 * G * 1536].reshape(nb4, G, 1536)
    groups = np.concatenate([f[:, :, :1024].reshape(nb4, G, 64, 16),
                             f[:, :, 1024:].reshape(nb4, G, 64, 8)], axis=-1)      # [b, c, lane, 24]
    vals = _fp6_ints(_codes_from_groups(groups))                                   # [b, c, lane, 32]
    vals = vals.reshape(nb4, G, 4, 16, 32)                                          # [b, c, g, n16, j]
    q[:, : nb4 * 128] = vals.transpose(1, 3, 0, 2, 4).reshape(N, nb4 * 128)
    f8 = WqF[nb4 * G * 1536:].reshape(nb8, G, 4, 16, 16)                            # [b, c, g, n16, j]
    lo = _sext4(f8 & 0xF)
    hi = _sext4(f8 >> 4)
    blk = np.stack([lo, hi], axis=4)                                                # [b, c, g, n16, half, j]
    q[:, nb4 * 128:] = blk.transpose(1, 3, 0, 2, 4, 5).reshape(N, nb8 * 128)
    return q


def pack_kv4_codes(u: np.ndarray) -> np.ndarray:
    """Codes uint8 [..., d] -> bytes [..., d/2]: channel 2i in the low nibble of
    byte i, 2i+1 in the high nibble."""
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_kv4_codes(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_kv4_codes."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def decode_xf(Xf: np.ndarray, M: int, nf: int) -> np.ndarray:
    """fp16 bits [M, nf] from the QUIK outlier tiles: tile (t, s) at half
    (t (nf/32) + s) 512, half 8l + e = row 16t + l mod 16, channel 32s + 8(l/16) + e."""
    steps = nf // 32
    mp = (M + 15) // 16 * 16
    h = np.asarray(Xf).view(np.uint16)[: mp * nf].reshape(mp // 16, steps, 4, 16, 8)   # t, s, l/16, l%16, e
    out = h.transpose(0, 3, 1, 2, 4).reshape(mp, nf)       # row = 16t + l%16, channel = 32s + 8(l/16) + e
    return out[:M]


def decode_wf(Wf: np.ndarray, N: int, nf: int) -> np.ndarray:
    """fp16 bits [N, nf] from the QUIK outlier weight fragments (same order as
    decode_xf with output channels for rows)."""
    return decode_xf(Wf, N, nf)
