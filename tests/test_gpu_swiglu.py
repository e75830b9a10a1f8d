"""GPU parity of the SwiGLU fused into the quantizer
(comet_swiglu_quant_act[_fp6]) and of the SwiGLU on its own (comet_swiglu),
through the C ABI against the CPU oracle.

Bit-exact: the fp16 rows fp16(silu(g) u), and the codes and scales of the
fused calls against the oracle's quantization of its own SwiGLU rows, on every
kernel path of the quantizer (row in LDS, element-wise staging of an
unaligned row stride, row in global memory for K > 32768), both layouts, with
the gate and up rows as the two halves of one projection output; and the
fused calls against SwiGLU-then-quantize on the GPU, byte for byte.
"""
import numpy as np
import pytest

from gen import synth
from tests import gpu_common as G
from tests.layout import decode_xq, decode_xq_fp6

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import w4ax_mixed_precision_amd as comet
    comet.lib()        # the HIP library must load: no fallback
    return t


def _inputs(M, K, seed):
    cfg = synth.LayerConfig("swiglu", M, K, 128, seed)
    g, u = synth.make_gate_up(cfg)
    # calibration-style score: per-channel absmax of the gate draw
    score = np.abs(g.view(np.float16).astype(np.float32)).max(axis=0)
    return g, u, score


def _halves(torch, g, u, ldx):
    """gate and up as the two halves of one [M, ldx] device tensor (ldx >= 2K),
    or of two padded tensors when ldx < 2K."""
    M, K = g.shape
    if ldx >= 2 * K:
        buf = np.zeros((M, ldx), np.uint16)
        buf[:, :K] = g
        buf[:, K:2 * K] = u
        d = torch.from_numpy(buf.view(np.float16)).cuda()
        return d[:, :K], d[:, K:2 * K]
    pads = []
    for a in (g, u):
        p = np.zeros((M, ldx), np.uint16)
        p[:, :K] = a
        pads.append(torch.from_numpy(p.view(np.float16)).cuda()[:, :K])
    return pads[0], pads[1]


@pytest.mark.parametrize("M,K,ldx", [(1, 128, 256), (3, 1000, 1000), (37, 4096, 4100), (64, 28672, 57344),
                                     (2, 33024, 33024)])
def test_swiglu_parity(torch, M, K, ldx):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[swiglu] M={M} K={K} ldx={ldx}")
    g, u, _ = _inputs(M, K, seed=M + K)
    want = O.swiglu(g, u)
    gd, ud = _halves(torch, g, u, ldx)
    out = torch.full((M, K + 8), 3.0, dtype=torch.float16, device="cuda")
    comet.comet_swiglu(gd, ud, K=K, H=out[:, :K])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got[:, :K].view(np.uint16), want)
    assert np.all(got[:, K:] == 3.0)                  # columns past K untouched


def test_swiglu_large_gates_and_ties(torch):
    """Gates above 36, where sigma(g) is 1 in binary64 and g u often sits on an
    fp16 midpoint (the true value rounds toward zero), plus zeros of both signs
    and gates far below zero."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    rng = np.random.default_rng(5)
    M, K = 4, 4096
    g = rng.integers(37, 2048, (M, K)).astype(np.float16)
    u = (rng.integers(-255, 256, (M, K)) / 64.0).astype(np.float16)
    g[0, :64] = np.float16([0.0, -0.0] * 32)
    g[1, :64] = -rng.integers(20, 60000, 64).astype(np.float16)
    g, u = g.view(np.uint16), u.view(np.uint16)
    want = O.swiglu(g, u)
    H = comet.comet_swiglu(torch.from_numpy(g.view(np.float16)).cuda(), torch.from_numpy(u.view(np.float16)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("uval", [1.0, -3.0, 0.7109375, 61.0])
def test_swiglu_every_gate_value(torch, uval):
    """Every finite fp16 gate value against one up value: the binary32 test
    and the binary64 fix-up together give the oracle's bits for the whole gate
    domain (the binary32 error bound depends on g only)."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    g = np.concatenate([np.arange(0, 0x7C00, dtype=np.uint16), np.arange(0x8000, 0xFC00, dtype=np.uint16)])
    gv = g.view(np.float16).astype(np.float64)
    keep = np.abs(gv * uval) < 60000.0                      # products inside the fp16 range
    g = g[keep][: (keep.sum() // 1024) * 1024].reshape(-1, 1024)
    u = np.full(g.shape, np.float16(uval).view(np.uint16), np.uint16)
    want = O.swiglu(g, u)
    H = comet.comet_swiglu(torch.from_numpy(g.view(np.float16)).cuda(), torch.from_numpy(u.view(np.float16)).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy().view(np.uint16), want)
    # the fused form on the same rows (identity permutation, all 4-bit blocks):
    # its codes equal the oracle's quantization of the oracle's rows
    perm = np.arange(1024, dtype=np.int32)
    qa, sa = O.quantize_activations(want, perm, np.zeros(8, np.uint8))
    Xq, xs = comet.comet_swiglu_quant_act(torch.from_numpy(g.view(np.float16)).cuda(),
                                          torch.from_numpy(u.view(np.float16)).cuda(),
                                          torch.from_numpy(perm).cuda(), 0)
    torch.cuda.synchronize()
    assert np.array_equal(decode_xq(Xq.cpu().numpy(), g.shape[0], 1024, 0), qa)
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32))


# (M, K, ldx, nb8): per-row kernel with the rows in LDS, element-wise staging
# (ldx not a multiple of 8), rows in global memory (K > 32768), the 70B
# down-projection width, and many rows
CASES = [(1, 128, 256, 0), (1, 128, 256, 1), (3, 640, 1280, 1), (17, 1024, 2048, 2), (9, 4096, 4100, 3),
         (5, 33024, 66048, 4), (40, 28672, 57344, 9), (300, 2048, 4096, 1)]


@pytest.mark.parametrize("fp6", [False, True])
@pytest.mark.parametrize("M,K,ldx,nb8", CASES)
def test_fused_swiglu_quant_parity(torch, M, K, ldx, nb8, fp6):
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    G.log(f"[swiglu quant] M={M} K={K} ldx={ldx} nb8={nb8} fp6={fp6}")
    g, u, score = _inputs(M, K, seed=5 * M + K + nb8)
    H = O.swiglu(g, u)
    perm, flags = O.channel_order(score, nb8)
    qa, sa = O.quantize_activations(H, perm, flags)
    gd, ud = _halves(torch, g, u, ldx)
    Xq, xs = comet.comet_swiglu_quant_act(gd, ud, torch.from_numpy(perm).cuda(), nb8, fp6=fp6)
    torch.cuda.synchronize()
    dec = decode_xq_fp6 if fp6 else decode_xq
    assert np.array_equal(dec(Xq.cpu().numpy(), M, K, nb8), qa), "codes differ"
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("fp6", [False, True])
def test_fused_swiglu_equals_unfused(torch, fp6):
    """comet_swiglu then comet_quant_act[_fp6] gives the same bytes as the
    fused call (the 70B down-projection input: 1024 tokens x 28672 channels,
    gate and up as halves of one output)."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    M, K, nb8 = 1024, 28672, 67
    g, u, score = _inputs(M, K, seed=91)
    perm, _ = O.channel_order(score, nb8)
    pd = torch.from_numpy(perm).cuda()
    gd, ud = _halves(torch, g, u, 2 * K)
    H = comet.comet_swiglu(gd, ud, K=K)
    q = comet.comet_quant_act_fp6 if fp6 else comet.comet_quant_act
    Xq_u, xs_u = q(H, pd, nb8)
    Xq_f, xs_f = comet.comet_swiglu_quant_act(gd, ud, pd, nb8, fp6=fp6)
    torch.cuda.synchronize()
    assert torch.equal(xs_u, xs_f)
    if fp6:
        a = decode_xq_fp6(Xq_u.cpu().numpy(), M, K, nb8)
        b = decode_xq_fp6(Xq_f.cpu().numpy(), M, K, nb8)
        assert np.array_equal(a, b)
    else:
        assert torch.equal(Xq_u, Xq_f)


@pytest.mark.parametrize("fp6", [False, True])
def test_swiglu_rows_of_undecided_values(torch, fp6):
    """A row where every value is an exact fp16 tie of g u with sigma = 1 in
    binary32 (g = 1025, u = 3: the true value 3075 (1 - e^-1025) rounds down
    to 3074), so the binary32 test decides none of them: more than a wave's
    queue holds, and the rest take the binary64 form directly. A second row
    is ordinary."""
    import w4ax_mixed_precision_amd as comet
    from oracle import oracle as O
    M, K, nb8 = 2, 28672, 9
    g, u, score = _inputs(M, K, seed=44)
    g[0] = np.float16(1025.0).view(np.uint16)
    u[0] = np.float16(3.0).view(np.uint16)
    H = O.swiglu(g, u)
    assert np.all(H[0] == np.float16(3074.0).view(np.uint16))
    perm, flags = O.channel_order(score, nb8)
    qa, sa = O.quantize_activations(H, perm, flags)
    gd, ud = _halves(torch, g, u, 2 * K)
    Hd = comet.comet_swiglu(gd, ud, K=K)
    Xq, xs = comet.comet_swiglu_quant_act(gd, ud, torch.from_numpy(perm).cuda(), nb8, fp6=fp6)
    torch.cuda.synchronize()
    assert np.array_equal(Hd.cpu().numpy().view(np.uint16), H)
    dec = decode_xq_fp6 if fp6 else decode_xq
    assert np.array_equal(dec(Xq.cpu().numpy(), M, K, nb8), qa)
    assert np.array_equal(xs.cpu().numpy().T.view(np.uint32), sa.view(np.uint32))
