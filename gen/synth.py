"""Seeded synthetic inputs for the W4Ax mixed-precision GEMM.

This module only draws numbers. It holds none of the method's arithmetic (no
permutation, no quantization, no GEMM): both the CPU oracle and the GPU path
receive the arrays it returns, so it is the one piece of code they share.

What it draws, and why (the shapes follow LLaMA linear layers):

* Activations X, fp16 [M, K]. Standard normal, with a seeded set of outlier
  channels multiplied across every token. The COMET article (mmssai.com,
  section "1.离群点分布规律的重定义") reports that activation outliers sit in
  about a tenth of the channels, so n_out = round(0.1 K). The QUIK blog
  (deep-paper.org/paper/2310.09259, section "挑战: 离群值问题") reports
  outliers up to ~100x the rest, hence multipliers of 20..100.
  The LLaMA-7B down-projection input is drawn heavy-tailed instead
  (Student-t, 3 degrees of freedom, no planted channels), following the QUIK
  blog's case study of the high-variance down_proj input (Figure 10 there).
* Weights W, fp16 [N, K], normal with standard deviation 0.02.
* Channel scores, f32 [K]: per-channel absmax over a separate 256-token
  calibration draw with the same outlier channels and multipliers, which is
  the offline calibration step of the QUIK blog ("第一步: 识别与重排").

Random numbers: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) used as a
counter-based generator: value i of sub-stream s under seed S is
mix64(key(S, s) + (i + 1) * 0x9E3779B97F4A7C15). Uniforms take the top 53
bits; normals use Box-Muller on consecutive uniform pairs. Everything is
rounded to fp16 with round-to-nearest-even (numpy's float16 cast).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Sub-stream ids of one configuration's seed.
STREAM_X = 1
STREAM_W = 2
STREAM_PICK = 3
STREAM_MULT = 4
STREAM_CALIB = 5
STREAM_CHI = 6          # chi-square draws of the Student-t activations
STREAM_CALIB_CHI = 7    # chi-square draws of the Student-t calibration batch
STREAM_GATE = 8         # gate projection outputs (SwiGLU input)
STREAM_UP = 9           # up projection outputs (SwiGLU input)
STREAM_Q = 10           # decode queries of the KV4 attention
STREAM_K = 11           # cached keys
STREAM_V = 12           # cached values

_CHUNK = 1 << 22        # values per generation chunk (bounds peak host memory)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(seed: int, stream: int) -> np.uint64:
    base = np.array([(seed * 0x100000001B3 + stream * 0x9E3779B1) & ((1 << 64) - 1)],
                    dtype=np.uint64)
    return _mix64(base)[0]


def u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Values start .. start+count-1 of sub-stream `stream` under `seed`."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(_key(seed, stream) + idx * GOLDEN_GAMMA)


def uniform(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    z = u64(seed, stream, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _normal_chunk(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Normals start .. start+count-1; value 2j/2j+1 come from uniform pair j."""
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = uniform(seed, stream, 2 * p0, 2 * (p1 - p0))
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    th = (2.0 * math.pi) * u2
    z = np.empty(2 * (p1 - p0), dtype=np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return z[off:off + count]


def normal(seed: int, stream: int, count: int, scale: float = 1.0,
           dtype=np.float64) -> np.ndarray:
    """`count` standard normals times `scale`, drawn chunk by chunk into `dtype`."""
    out = np.empty(count, dtype=dtype)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = (_normal_chunk(seed, stream, s, n) * scale).astype(dtype)
    return out


def student_t3(seed: int, stream_z: int, stream_chi: int, count: int,
               dtype=np.float64) -> np.ndarray:
    """Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    out = np.empty(count, dtype=dtype)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        z = _normal_chunk(seed, stream_z, s, n)
        c = _normal_chunk(seed, stream_chi, 3 * s, 3 * n).reshape(n, 3)
        chi2 = (c * c).sum(axis=1)
        out[s:s + n] = (z / np.sqrt(chi2 / 3.0)).astype(dtype)
    return out


def pick_channels(seed: int, K: int, n_out: int) -> np.ndarray:
    """n_out distinct channels of [0, K): first n_out steps of a Fisher-Yates shuffle."""
    idx = np.arange(K, dtype=np.int64)
    u = uniform(seed, STREAM_PICK, 0, max(n_out, 1))
    for i in range(n_out):
        j = i + int(u[i] * (K - i))
        idx[i], idx[j] = idx[j], idx[i]
    return np.sort(idx[:n_out])


def multipliers(seed: int, n_out: int, kind: str, lo: float, hi: float) -> np.ndarray:
    if kind == "const":
        return np.full(n_out, lo, dtype=np.float64)
    if kind == "loguniform":
        u = uniform(seed, STREAM_MULT, 0, n_out)
        return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    raise ValueError(kind)


def to_fp16(a: np.ndarray) -> np.ndarray:
    """Round to IEEE binary16, nearest-even; the fp16 bit patterns as uint16.

    Values are first clipped to the largest finite fp16 magnitude, so that a
    rare heavy-tail draw stays finite."""
    a = np.clip(np.asarray(a, dtype=np.float32), -65504.0, 65504.0)
    return a.astype(np.float16).view(np.uint16)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One synthetic linear layer: Y[M, N] = X[M, K] W[N, K]^T."""
    name: str
    M: int
    K: int
    N: int
    seed: int
    x_kind: str = "planted"         # "planted" or "student_t"
    mult_kind: str = "const"        # outlier multiplier law
    mult_lo: float = 50.0
    mult_hi: float = 50.0
    int8_frac: float | None = None  # fraction of INT8 blocks, if stated
    calib_tokens: int = 256

    @property
    def nb(self) -> int:
        return self.K // 128

    @property
    def n_out(self) -> int:
        if self.x_kind != "planted":
            return 0
        return int(math.floor(0.1 * self.K + 0.5))

    @property
    def nb8(self) -> int:
        if self.int8_frac is not None:
            return int(math.floor(self.int8_frac * self.nb + 0.5))
        return -(-self.n_out // 128)

    def with_m(self, M: int, name: str | None = None) -> "LayerConfig":
        return dataclasses.replace(self, M=M, name=name or f"{self.name}_m{M}")


def _layers() -> dict[str, LayerConfig]:
    c = {}
    c["tiny"] = LayerConfig("tiny", 16, 512, 512, 1001)
    c["q_proj_7b"] = LayerConfig("q_proj_7b", 128, 4096, 4096, 1002,
                                 mult_kind="loguniform", mult_lo=20.0, mult_hi=100.0)
    c["up_gate_7b"] = LayerConfig("up_gate_7b", 1024, 4096, 11008, 1003,
                                  mult_kind="loguniform", mult_lo=20.0, mult_hi=100.0)
    c["down_7b"] = LayerConfig("down_7b", 1024, 11008, 4096, 1013,
                               x_kind="student_t", int8_frac=0.25)
    for n in (10240, 8192, 28672):
        for m in (1, 4, 16, 64):
            nm = f"decode_70b_n{n}_m{m}"
            c[nm] = LayerConfig(nm, m, 8192, n, 1004)
    c["prefill_down_70b"] = LayerConfig("prefill_down_70b", 4096, 28672, 8192, 1005,
                                        int8_frac=0.30)
    c["prefill_up_70b"] = LayerConfig("prefill_up_70b", 4096, 8192, 28672, 1015)
    return c


CONFIGS: dict[str, LayerConfig] = _layers()


def outlier_plan(cfg: LayerConfig) -> tuple[np.ndarray, np.ndarray]:
    """(outlier channel indices, their multipliers) of a configuration."""
    ch = pick_channels(cfg.seed, cfg.K, cfg.n_out)
    mu = multipliers(cfg.seed, cfg.n_out, cfg.mult_kind, cfg.mult_lo, cfg.mult_hi)
    return ch, mu


def _activations(cfg: LayerConfig, M: int, stream: int, chi_stream: int) -> np.ndarray:
    K = cfg.K
    if cfg.x_kind == "student_t":
        x = student_t3(cfg.seed, stream, chi_stream, M * K, dtype=np.float32)
        return x.reshape(M, K)
    x = normal(cfg.seed, stream, M * K, dtype=np.float32).reshape(M, K)
    ch, mu = outlier_plan(cfg)
    if len(ch):
        x[:, ch] *= mu.astype(np.float32)[None, :]
    return x


def make_x(cfg: LayerConfig, rows: int | None = None) -> np.ndarray:
    """Activations as fp16 bit patterns, uint16 [M, K]. `rows` draws only the first rows."""
    M = cfg.M if rows is None else rows
    return to_fp16(_activations(cfg, M, STREAM_X, STREAM_CHI))


def make_w(cfg: LayerConfig) -> np.ndarray:
    """Weights as fp16 bit patterns, uint16 [N, K], drawn N(0, 0.02^2)."""
    w = normal(cfg.seed, STREAM_W, cfg.N * cfg.K, scale=0.02, dtype=np.float32)
    return to_fp16(w).reshape(cfg.N, cfg.K)


def make_scores(cfg: LayerConfig) -> np.ndarray:
    """Per-channel absmax of the fp16-rounded calibration batch, f32 [K]."""
    cal = _activations(cfg, cfg.calib_tokens, STREAM_CALIB, STREAM_CALIB_CHI)
    cal16 = to_fp16(cal).view(np.float16).astype(np.float32)
    return np.abs(cal16).max(axis=0).astype(np.float32)


def make_gate_up(cfg: LayerConfig, rows: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """The gate and up projection outputs that feed the down projection's
    SwiGLU, fp16 bit patterns [M, K] each (K = the down projection's input
    width). Gate: normal with standard deviation 2 and the configuration's
    outlier channels multiplied by its 20..100 factors, so a few channels
    carry the large values the down projection's input is known for (QUIK
    blog, Figure 10 of its down-projection case study); up: standard normal.
    The up value is clipped to |u| <= 16384 / max(|g|, 1), which keeps every
    product |g u| inside the fp16 range."""
    M = cfg.M if rows is None else rows
    K = cfg.K
    g = normal(cfg.seed, STREAM_GATE, M * K, scale=2.0, dtype=np.float32).reshape(M, K)
    ch, mu = outlier_plan(cfg)
    if len(ch):
        g[:, ch] *= mu.astype(np.float32)[None, :]
    g16 = to_fp16(g)
    gv = np.abs(g16.view(np.float16).astype(np.float32))
    u = normal(cfg.seed, STREAM_UP, M * K, dtype=np.float32).reshape(M, K)
    cap = 16384.0 / np.maximum(gv, 1.0)
    return g16, to_fp16(np.clip(u, -cap, cap))


def make_layer(cfg: LayerConfig) -> dict:
    """All inputs of one configuration."""
    return {"X": make_x(cfg), "W": make_w(cfg), "score": make_scores(cfg),
            "nb8": cfg.nb8, "cfg": cfg}


def fp16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)


def make_kv(seed: int, ntok: int, H: int, d: int, Hq: int | None = None):
    """Inputs of KV4 decode attention, fp16 bit patterns: queries [Hq, d] ~ N(0, 1),
    keys and values [ntok, H d] (token rows, heads side by side, as the key and
    value projections write them). Values ~ N(0, 1); keys ~ N(0, 1) with d / 16
    outlier channels per head (channels 16 i + 3) scaled by 8, the fixed
    large-magnitude key channels that make per-channel ranges uneven."""
    Hq = H if Hq is None else Hq
    q = normal(seed, STREAM_Q, Hq * d, dtype=np.float32).reshape(Hq, d)
    k = normal(seed, STREAM_K, ntok * H * d, dtype=np.float32).reshape(ntok, H, d)
    k[:, :, 3::16] *= 8.0
    v = normal(seed, STREAM_V, ntok * H * d, dtype=np.float32).reshape(ntok, H * d)
    return to_fp16(q), to_fp16(k.reshape(ntok, H * d)), to_fp16(v)
