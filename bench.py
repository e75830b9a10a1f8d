"""Benchmark of the W4Ax mixed-precision linear layer on one MI355X.

A step is one pass of the online path over one batch of synthetic input:
comet_quant_act then comet_w4ax_gemm, for every layer of the workload. The
offline steps (channel ranking, weight quantization and packing) run once
before timing, as the method prescribes for static weights.

Default workload: the LLaMA-70B prefill pair, 4096 tokens, down_proj
(K = 28672 -> N = 8192, 30% 8-bit blocks) and up_proj (K = 8192 -> N = 28672,
7 of 64 blocks 8-bit). `--workload decode_70b` times the decode sweep
(M in {1, 4, 16, 64} x N in {10240, 8192, 28672}, K = 8192).

Prints one JSON line. `value` is effective TOPS: 2 M N K per layer, summed,
over the measured step time. The roofline object is for comet_w4ax_gemm, the
dominant kernel, from HIP events recorded around its launches on the stream
they run on. Its `traffic` is the HBM bytes of one step's GEMM launches taken
from hardware counters (FETCH_SIZE and WRITE_SIZE, scaled by what the same
counters read for a device copy of known size), read from the counter summary
under profiles/ when that summary was taken on the current kernel sources,
otherwise null. `--copy-calibration` runs only that known-size copy.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, published
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
STREAM_MAX_M = 64            # the library's INT4-layout GEMM streams weights up to this M

WORKLOADS = {
    "prefill_70b": ["prefill_down_70b", "prefill_up_70b"],
    "decode_70b": [f"decode_70b_n{n}_m{m}" for n in (10240, 8192, 28672) for m in (1, 4, 16, 64)],
    "q_proj_7b": ["q_proj_7b"],
    "mlp_7b": ["up_gate_7b", "down_7b"],
}


# Sources whose change invalidates counter data taken on the GEMM kernels of
# a workload: the GEMM source of the layout the workload runs and what every
# kernel includes; the compiler flags are hashed with them.
_COMMON_SOURCES = ["w4ax_mixed_precision_amd/csrc/device_util.h",
                   "w4ax_mixed_precision_amd/csrc/comet_internal.h"]
KERNEL_SOURCES = {"int4": ["w4ax_mixed_precision_amd/csrc/w4ax_gemm.hip"] + _COMMON_SOURCES,
                  "fp6": ["w4ax_mixed_precision_amd/csrc/w4ax_gemm_fp6.hip"] + _COMMON_SOURCES}
COPY_CAL_BYTES = 1 << 30


def workload_layouts(workload):
    return sorted({layout_of(synth_cfg(n).M) for n in WORKLOADS[workload]})


def synth_cfg(name):
    from gen import synth
    return synth.CONFIGS[name]


def kernel_sources_digest(workload):
    from w4ax_mixed_precision_amd import build as _b
    h = hashlib.sha256(repr(_b.FLAGS).encode())
    for rel in [r for lay in workload_layouts(workload) for r in KERNEL_SOURCES[lay]]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per step of the GEMM launches from the committed counter summary
    of this workload, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"w4ax_gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha256") != kernel_sources_digest(workload):
        return None, "kernel changed since the counters were taken"
    return float(rec["hbm_bytes_per_step"]), path


def copy_calibration(torch):
    """A plain device copy of COPY_CAL_BYTES, three times, for counter scaling."""
    n = COPY_CAL_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_CAL_BYTES, "copies": 3}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def layout_of(M):
    """INT4 layout (weight streaming) for decode shapes, FP6 layout above."""
    return "int4" if M <= STREAM_MAX_M else "fp6"


def gemm_bytes(M, N, K, nb8, layout):
    """Bytes one GEMM must move in its layout: weight codes, weight scales (and
    sums on the INT4 layout), activation codes and scales, fp16 output."""
    nb = K // 128
    nb4 = nb - nb8
    if layout == "int4":
        return N * K // 2 + 2 * N * nb + 2 * N * nb4 + M * (64 * nb4 + 128 * nb8) + 4 * M * nb + 2 * M * N
    return N * (96 * nb4 + 64 * nb8) + 2 * N * nb + M * (96 * nb4 + 128 * nb8) + 4 * M * nb + 2 * M * N


def gemm_peak_tops(M, N, K, nb8, layout):
    """Dense matrix-unit peak for this GEMM's instruction mix: INT8 for every
    block on the INT4 layout; FP6 for the 4-bit blocks and INT8 for the 8-bit
    blocks on the FP6 layout."""
    nb = K // 128
    if layout == "int4":
        return PEAK_INT8_TOPS
    nb4 = nb - nb8
    return 1.0 / ((nb4 / PEAK_FP6_TOPS + nb8 / PEAK_INT8_TOPS) / nb)


def quant_bytes(M, K, nb8, layout):
    nb = K // 128
    nb4 = nb - nb8
    per4 = 64 if layout == "int4" else 96
    return 2 * M * K + 4 * K + M * (per4 * nb4 + 128 * nb8) + 4 * M * nb


class Layer:
    def __init__(self, name, copies, torch, comet, synth):
        cfg = synth.CONFIGS[name]
        self.cfg = cfg
        self.name = name
        t0 = time.time()
        X, W, score = synth.make_x(cfg), synth.make_w(cfg), synth.make_scores(cfg)
        self.host = {"X": X, "W": W, "score": score}
        self.layout = layout_of(cfg.M)
        pk = comet.comet_pack_weights(W, score, cfg.nb8)
        if self.layout == "fp6":
            comet.comet_repack_weights_fp6(pk)
            pk.pop("Wq")                        # keep only the layout this layer runs
        self.pk = pk
        w = comet.upload_weights(pk)
        self.w = [w] + [{k: (v.clone() if hasattr(v, "clone") else v) for k, v in w.items()}
                        for _ in range(copies - 1)]
        self.X = torch.from_numpy(X.view(np.float16)).cuda()
        M, K, N = cfg.M, cfg.K, cfg.N
        nxq = comet.xq_bytes(M, K, cfg.nb8) if self.layout == "int4" else comet.xq_fp6_bytes(M, K, cfg.nb8)
        self.Xq = torch.empty(nxq, dtype=torch.uint8, device="cuda")
        self.xs = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
        self.Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        need = (comet.workspace_bytes(M, N, K, cfg.nb8) if self.layout == "int4"
                else comet.fp6_workspace_bytes(M, N, K, cfg.nb8))
        # zeroed once: the library leaves it zeroed after every call
        self.ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda") if need else None
        self.ws_bytes = need
        self.ops = 2.0 * M * N * K
        self.gbytes = gemm_bytes(M, N, K, cfg.nb8, self.layout)
        self.qbytes = quant_bytes(M, K, cfg.nb8, self.layout)
        self.peak = gemm_peak_tops(M, N, K, cfg.nb8, self.layout)
        log(f"[bench] {name}: M={M} K={K} N={N} nb8={cfg.nb8} {self.layout} layout, ready in "
            f"{time.time() - t0:.1f}s ({copies} weight copies)")

    def quant(self, w):
        import w4ax_mixed_precision_amd as comet
        if self.layout == "int4":
            comet.comet_quant_act(self.X, w["perm"], self.cfg.nb8, Xq=self.Xq, x_scale=self.xs)
        else:
            comet.comet_quant_act_fp6(self.X, w["perm"], self.cfg.nb8, Xq=self.Xq, x_scale=self.xs)

    def gemm(self, w):
        import w4ax_mixed_precision_amd as comet
        if self.layout == "int4":
            comet.comet_w4ax_gemm(self.Xq, self.xs, w, self.cfg.M, Y=self.Y, workspace=self.ws)
        else:
            comet.comet_w4ax_gemm_fp6(self.Xq, self.xs, w, self.cfg.M, Y=self.Y, workspace=self.ws)


def copies_for(cfg, target_bytes=1 << 30):
    nb = cfg.K // 128
    per = gemm_bytes(0, cfg.N, cfg.K, cfg.nb8, layout_of(cfg.M)) - 2 * cfg.N * nb
    return int(max(1, min(32, -(-target_bytes // per))))


def run_gpu(layers, steps, warmup, torch, comet):
    """Warm up, then time exactly `steps` steps between two synchronizations.
    Events recorded on the launch stream around every launch give the per-kernel
    durations inside the same timed region."""
    ev = {l.name: [] for l in layers}
    qev = {l.name: [] for l in layers}

    def step(i, record):
        for l in layers:
            w = l.w[i % len(l.w)]
            if record:
                a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                a.record()
            l.quant(w)
            if record:
                b.record()
            l.gemm(w)
            if record:
                c.record()
                qev[l.name].append((a, b))
                ev[l.name].append((b, c))

    for i in range(warmup):
        step(i, False)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i, True)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    per = {}
    for l in layers:
        g = [a.elapsed_time(b) for a, b in ev[l.name]]
        q = [a.elapsed_time(b) for a, b in qev[l.name]]
        per[l.name] = {"gemm_ms": float(np.mean(g)), "gemm_ms_p10": float(np.percentile(g, 10)),
                       "gemm_ms_p90": float(np.percentile(g, 90)), "quant_ms": float(np.mean(q))}
    return step_ms, per


def _time_variants(torch, variants, iters):
    """Mean microseconds per call of each (name, fn): HIP events on the launch
    stream around `iters` back-to-back calls, after 3 untimed ones."""
    res = {}
    for name, fn in variants:
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / iters
    return res


def swiglu_ablation(torch, comet, synth, M=4096, K=28672, nb8=67, iters=10):
    """The quantizer fused into the SwiGLU before it, against the two steps
    apart (comet_swiglu, then comet_quant_act_fp6), at the 70B down-projection
    input (4096 tokens x 28672 channels; gate and up as the two halves of one
    [M, 2K] projection output)."""
    cfg = synth.LayerConfig("swiglu_quant_70b", M, K, 128, 29)
    g16, u16 = synth.make_gate_up(cfg)
    gu = torch.empty((M, 2 * K), dtype=torch.float16, device="cuda")
    gu[:, :K] = torch.from_numpy(g16.view(np.float16)).cuda()
    gu[:, K:] = torch.from_numpy(u16.view(np.float16)).cuda()
    del g16, u16
    gate, up = gu[:, :K], gu[:, K:]
    perm = np.random.default_rng(29).permutation(K).astype(np.int32)   # any permutation serves for timing
    pd = torch.from_numpy(perm).cuda()
    H = torch.empty((M, K), dtype=torch.float16, device="cuda")
    Xq = torch.empty(comet.xq_fp6_bytes(M, K, nb8), dtype=torch.uint8, device="cuda")
    xs = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")

    def unfused():
        comet.comet_swiglu(gate, up, K=K, H=H)
        comet.comet_quant_act_fp6(H, pd, nb8, Xq=Xq, x_scale=xs)

    def fused():
        comet.comet_swiglu_quant_act(gate, up, pd, nb8, Xq=Xq, x_scale=xs, fp6=True)

    res = _time_variants(torch, (("unfused", unfused), ("fused", fused)), iters)
    codes = M * (96 * (K // 128 - nb8) + 128 * nb8) + 4 * M * (K // 128)
    hbytes = 2 * M * K
    return {"shape": {"M": M, "K": K, "int8_blocks": nb8, "layout": "fp6"},
            "unfused_us": res["unfused"], "fused_us": res["fused"],
            "speedup": res["unfused"] / res["fused"],
            "hbm_bytes_unfused": 4 * hbytes + codes, "hbm_bytes_fused": 2 * hbytes + codes,
            "fused_gbs": (2 * hbytes + codes) / (res["fused"] * 1e-6) / 1e9,
            "timing": f"HIP events around {iters} back-to-back iterations of each variant"}


def fusion_ablation(torch, comet, synth, M=4096, K=8192, nb8=7, iters=20):
    """The quantizer fused into the RMS normalization before it, against the two
    steps apart (comet_rmsnorm, then comet_quant_act_fp6), at the 70B up/gate
    input (4096 tokens x 8192 channels). HIP events on the launch stream around
    `iters` back-to-back iterations of each variant."""
    cfg = synth.LayerConfig("norm_quant_70b", M, K, 128, 17)
    X = torch.from_numpy(synth.make_x(cfg).view(np.float16)).cuda()
    rng = np.random.default_rng(17)
    gamma16 = synth.to_fp16(1.0 + 0.25 * rng.standard_normal(K))
    score = synth.make_scores(cfg)
    perm = np.argsort(score, kind="stable").astype(np.int32)     # any permutation serves for timing
    gamma = torch.from_numpy(gamma16.view(np.float16)).cuda()
    gperm = torch.from_numpy(comet.comet_permute_channels(gamma16, perm).view(np.float16)).cuda()
    pd = torch.from_numpy(perm).cuda()
    Xn = torch.empty((M, K), dtype=torch.float16, device="cuda")
    Xq = torch.empty(comet.xq_fp6_bytes(M, K, nb8), dtype=torch.uint8, device="cuda")
    xs = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")

    def unfused():
        comet.comet_rmsnorm(X, gamma, 1e-5, Xn=Xn)
        comet.comet_quant_act_fp6(Xn, pd, nb8, Xq=Xq, x_scale=xs)

    def fused():
        comet.comet_rmsnorm_quant_act(X, gperm, 1e-5, pd, nb8, Xq=Xq, x_scale=xs, fp6=True)

    res = _time_variants(torch, (("unfused", unfused), ("fused", fused)), iters)
    codes = M * (96 * (K // 128 - nb8) + 128 * nb8) + 4 * M * (K // 128)
    xbytes = 2 * M * K
    return {"shape": {"M": M, "K": K, "int8_blocks": nb8, "layout": "fp6"},
            "unfused_us": res["unfused"], "fused_us": res["fused"],
            "speedup": res["unfused"] / res["fused"],
            "hbm_bytes_unfused": 3 * xbytes + codes, "hbm_bytes_fused": xbytes + codes,
            "fused_gbs": (xbytes + codes) / (res["fused"] * 1e-6) / 1e9,
            "timing": f"HIP events around {iters} back-to-back iterations of each variant"}


def asym_ablation(torch, comet, synth, Ms=(1, 16, 64, 4096), iters=20):
    """Asymmetric 4-bit activation blocks (scale and zero point) against the
    symmetric ones, both on the INT4 layout, at the LLaMA-70B up_proj shape
    (K = 8192, N = 28672, 7 of 64 blocks 8-bit): quantizer + GEMM per M (the
    streaming kernels for M <= 64, the tiled INT8 kernel above), HIP events
    around `iters` back-to-back iterations over weight copies of >= 1 GB; and
    the error of each against the unquantized product X W^T on 16 rows."""
    cfg0 = synth.CONFIGS["prefill_up_70b"]
    K, N, nb8 = cfg0.K, cfg0.N, cfg0.nb8
    W, score = synth.make_w(cfg0), synth.make_scores(cfg0)
    pk = comet.comet_pack_weights(W, score, nb8)
    w0 = comet.upload_weights(pk)
    copies = copies_for(synth.LayerConfig("asym", 1, K, N, 0, int8_frac=None))
    ws = [w0] + [{k: (v.clone() if hasattr(v, "clone") else v) for k, v in w0.items()} for _ in range(copies - 1)]
    Xall = synth.make_x(cfg0)
    out = {"shape": {"K": K, "N": N, "int8_blocks": nb8, "layout": "int4"}, "per_M": {},
           "timing": f"HIP events around {iters} back-to-back quantizer + GEMM pairs, {copies} weight copies"}
    for M in Ms:
        X = torch.from_numpy(Xall[:M].view(np.float16)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        Xq = torch.empty(comet.xq_bytes(M, K, nb8), dtype=torch.uint8, device="cuda")
        xs = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
        xz = torch.zeros((K // 128, (M + 15) // 16 * 16), dtype=torch.uint8, device="cuda")
        it = {"i": 0}

        def sym():
            w = ws[it["i"] % copies]
            it["i"] += 1
            comet.comet_quant_act(X, w["perm"], nb8, Xq=Xq, x_scale=xs)
            comet.comet_w4ax_gemm(Xq, xs, w, M, Y=Y)

        def asym():
            w = ws[it["i"] % copies]
            it["i"] += 1
            comet.comet_quant_act_asym(X, w["perm"], nb8, Xq=Xq, x_scale=xs, x_zero=xz)
            comet.comet_w4ax_gemm_asym(Xq, xs, xz, w, M, Y=Y)

        res = _time_variants(torch, (("sym", sym), ("asym", asym)), iters if M <= 64 else 5)
        out["per_M"][str(M)] = {"sym_us": res["sym"], "asym_us": res["asym"],
                                "asym_over_sym": res["asym"] / res["sym"]}
    # error against the unquantized product on 16 planted-outlier rows
    rows = 16
    X = torch.from_numpy(Xall[:rows].view(np.float16)).cuda()
    ref = Xall[:rows].view(np.float16).astype(np.float64) @ W.view(np.float16).astype(np.float64).T
    err = {}
    for name in ("sym", "asym"):
        if name == "sym":
            Xq, xs = comet.comet_quant_act(X, w0["perm"], nb8)
            Y = comet.comet_w4ax_gemm(Xq, xs, w0, rows)
        else:
            Xq, xs, xz = comet.comet_quant_act_asym(X, w0["perm"], nb8)
            Y = comet.comet_w4ax_gemm_asym(Xq, xs, xz, w0, rows)
        y = Y.float().cpu().numpy().astype(np.float64)
        err[name] = float(np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    out["rel_rms_err_vs_unquantized"] = err
    del ws
    torch.cuda.empty_cache()
    return out


def quik_ablation(torch, comet, synth, Ms=(16, 4096), iters=20):
    """QUIK's split (the top nf channels in fp16 on their own path, every other
    block 4-bit) against the COMET form (the same layer with its 8-bit
    blocks), all on the FP6 layout, at the LLaMA-70B up_proj shape (K = 8192,
    N = 28672, 7 8-bit blocks): nf = 896 keeps exactly the channels of the 8-bit
    blocks in fp16, nf = 256 is QUIK's usual outlier count. Quantizer + GEMM,
    HIP events around `iters` back-to-back pairs over weight copies of >= 1 GB;
    and each one's error against the unquantized product on 16 rows."""
    cfg0 = synth.CONFIGS["prefill_up_70b"]
    K, N, nb8 = cfg0.K, cfg0.N, cfg0.nb8
    W, score = synth.make_w(cfg0), synth.make_scores(cfg0)
    copies = copies_for(synth.LayerConfig("quik", 1, K, N, 0, int8_frac=None))

    def clone(w):
        return {k: (v.clone() if hasattr(v, "clone") else v) for k, v in w.items()}

    def replicas(w0):
        return [w0] + [clone(w0) for _ in range(copies - 1)]
    variants = {"comet": (replicas(comet.upload_weights(
        comet.comet_repack_weights_fp6(comet.comet_pack_weights(W, score, nb8)))), 0)}
    for nf in (128 * nb8, 256):
        variants[f"quik_nf{nf}"] = (replicas(comet.upload_weights(comet.comet_pack_weights_quik(W, score, 0, nf))), nf)
    Xall = synth.make_x(cfg0)
    out = {"shape": {"K": K, "N": N, "comet_int8_blocks": nb8, "layout": "fp6"}, "per_M": {},
           "timing": f"HIP events around {iters} back-to-back quantizer + GEMM pairs, {copies} weight copies"}

    def pair(name, X, M, Y, i):
        ws, nf = variants[name]
        w = ws[i % copies]
        if nf == 0:
            Xq, xs = comet.comet_quant_act_fp6(X, w["perm"], nb8)
            return comet.comet_w4ax_gemm_fp6(Xq, xs, w, M, Y=Y)
        Xq, xs, Xf = comet.comet_quant_act_quik_fp6(X, w["perm"], 0, nf)
        return comet.comet_w4ax_gemm_quik_fp6(Xq, xs, Xf, w, M, Y=Y)

    for M in Ms:
        X = torch.from_numpy(Xall[:M].view(np.float16)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fns = []
        for name in variants:
            it = {"i": 0}

            def fn(name=name, it=it):
                pair(name, X, M, Y, it["i"])
                it["i"] += 1
            fns.append((name, fn))
        res = _time_variants(torch, fns, iters if M <= 64 else 5)
        out["per_M"][str(M)] = {f"{k}_us": v for k, v in res.items()}
    rows = 16
    X = torch.from_numpy(Xall[:rows].view(np.float16)).cuda()
    ref = Xall[:rows].view(np.float16).astype(np.float64) @ W.view(np.float16).astype(np.float64).T
    err = {}
    for name in variants:
        y = pair(name, X, rows, None, 0).float().cpu().numpy().astype(np.float64)
        err[name] = float(np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2)))
    out["rel_rms_err_vs_unquantized"] = err
    del variants
    torch.cuda.empty_cache()
    return out


def qoq_ablation(torch, comet, synth, Ms=(1, 16, 64, 4096), iters=20):
    """QoQ's W4A8 variant (per-channel INT8 then per-group UINT4 weights;
    per-token INT8 activations; one integer sum over K) against the W4Ax path
    on the INT4 layout (its tiled INT8 kernel for M > 64), at the LLaMA-70B
    up_proj shape (K = 8192, N = 28672) for decode row counts and 4096 rows:
    quantizer + GEMM, HIP events around `iters` back-to-back pairs over weight
    copies of >= 1 GB; and each one's error against the unquantized product on
    16 rows."""
    cfg0 = synth.CONFIGS["prefill_up_70b"]
    K, N, nb8 = cfg0.K, cfg0.N, cfg0.nb8
    W, score = synth.make_w(cfg0), synth.make_scores(cfg0)
    w4 = comet.upload_weights(comet.comet_pack_weights(W, score, nb8))
    wq = comet.upload_qoq(comet.comet_pack_weights_qoq(W, score))
    copies = copies_for(synth.LayerConfig("qoq", 1, K, N, 0, int8_frac=None))
    clone = lambda w: {k: (v.clone() if hasattr(v, "clone") else v) for k, v in w.items()}
    w4s = [w4] + [clone(w4) for _ in range(copies - 1)]
    wqs = [wq] + [clone(wq) for _ in range(copies - 1)]
    Xall = synth.make_x(cfg0)
    out = {"shape": {"K": K, "N": N, "int8_blocks_w4ax": nb8}, "per_M": {},
           "timing": f"HIP events around {iters} back-to-back quantizer + GEMM pairs, {copies} weight copies"}
    for M in Ms:
        X = torch.from_numpy(Xall[:M].view(np.float16)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        Xq4 = torch.empty(comet.xq_bytes(M, K, nb8), dtype=torch.uint8, device="cuda")
        xs4 = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
        Xq8 = torch.empty(M * K, dtype=torch.uint8, device="cuda")
        xs8 = torch.empty(M, dtype=torch.float32, device="cuda")
        it = {"i": 0}

        def w4ax():
            w = w4s[it["i"] % copies]
            it["i"] += 1
            comet.comet_quant_act(X, w["perm"], nb8, Xq=Xq4, x_scale=xs4)
            comet.comet_w4ax_gemm(Xq4, xs4, w, M, Y=Y)

        def qoq():
            w = wqs[it["i"] % copies]
            it["i"] += 1
            comet.comet_quant_act_token_i8(X, w["perm"], Xq=Xq8, x_scale=xs8)
            comet.comet_w4a8_qoq_gemm(Xq8, xs8, w, M, Y=Y)

        res = _time_variants(torch, (("w4ax", w4ax), ("qoq", qoq)), iters if M <= 64 else 5)
        out["per_M"][str(M)] = {"w4ax_us": res["w4ax"], "qoq_us": res["qoq"],
                                "qoq_over_w4ax": res["qoq"] / res["w4ax"]}
    rows = 16
    X = torch.from_numpy(Xall[:rows].view(np.float16)).cuda()
    ref = Xall[:rows].view(np.float16).astype(np.float64) @ W.view(np.float16).astype(np.float64).T
    Xq, xs = comet.comet_quant_act(X, w4["perm"], nb8)
    y4 = comet.comet_w4ax_gemm(Xq, xs, w4, rows).float().cpu().numpy().astype(np.float64)
    Xq, xs = comet.comet_quant_act_token_i8(X, wq["perm"])
    yq = comet.comet_w4a8_qoq_gemm(Xq, xs, wq, rows).float().cpu().numpy().astype(np.float64)
    nrm = np.sqrt(np.mean(ref ** 2))
    out["rel_rms_err_vs_unquantized"] = {"w4ax": float(np.sqrt(np.mean((y4 - ref) ** 2)) / nrm),
                                         "qoq": float(np.sqrt(np.mean((yq - ref) ** 2)) / nrm)}
    del w4s, wqs
    torch.cuda.empty_cache()
    return out


def kv4_attention_measure(torch, comet, synth, T=4096, seqs=16, iters=20):
    """KV4 decode attention (4-bit keys and values with an fp16 step and zero
    point per head and token) for `seqs` sequences of T cached tokens, d = 128:
    LLaMA-7B (32 heads, multi-head) and LLaMA-70B (64 query heads over 8 kv
    heads). HIP events around `iters` back-to-back calls over cache copies that
    together exceed the last-level cache. Algorithmic bytes: every cached code,
    step and zero point of K and V read once, plus q and the fp16 output."""
    out = {"timing": f"HIP events around {iters} back-to-back calls (split kernel + combine) queued behind an "
                     f"untimed one, median of 5 rounds, after 300 untimed calls",
           "shapes": {}}
    d = 128
    for name, hq_seq, group in (("llama7b_mha", 32, 1), ("llama70b_gqa8", 64, 8)):
        Hq = seqs * hq_seq
        H = Hq // group
        q16, K16, V16 = synth.make_kv(77, T, H, d, Hq)
        per_cache = H * T * (d // 2 + 3)
        copies = max(1, -(-(1 << 30) // (2 * per_cache)))
        caches = []
        X = torch.from_numpy(K16.view(np.float16)).cuda()
        Xv = torch.from_numpy(V16.view(np.float16)).cuda()
        for _ in range(copies):
            kc, vc = comet.kv4_cache(H, T, d), comet.kv4_cache(H, T, d)
            comet.comet_kv4_quantize(X, kc, 0)
            comet.comet_kv4_quantize(Xv, vc, 0)
            caches.append((kc, vc))
        del X, Xv
        q = torch.from_numpy(q16.view(np.float16)).cuda()
        o = torch.empty((Hq, d), dtype=torch.float16, device="cuda")
        ws = torch.empty(comet.lib().comet_kv4_attention_workspace_bytes(Hq, d, T), dtype=torch.uint8,
                         device="cuda")
        it = {"i": 0}

        def att():
            kc, vc = caches[it["i"] % copies]
            it["i"] += 1
            comet.comet_kv4_attention(q, kc, vc, T, group, out=o, workspace=ws)

        us = _median_us(torch, att, iters)
        nbytes = 2 * per_cache + 2 * Hq * d * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        out["shapes"][name] = {"query_heads": Hq, "kv_heads": H, "T": T, "d": d, "us": us,
                               "algorithmic_bytes": nbytes, "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                               "cache_copies": copies}
        # the same batch with the sequences at different positions (a decode
        # batch): lengths drawn uniformly from [T/8, T] per sequence, one call
        seq_T = np.random.default_rng(78).integers(T // 8, T + 1, size=seqs).astype(np.int32)
        Tkv = torch.from_numpy(np.repeat(seq_T, H // seqs)).cuda()

        def att_var():
            kc, vc = caches[it["i"] % copies]
            it["i"] += 1
            comet.comet_kv4_attention_varlen(q, kc, vc, Tkv, T, group, out=o, workspace=ws)

        usv = _median_us(torch, att_var, iters)
        vbytes = 2 * (H // seqs) * int(seq_T.sum()) * (d // 2 + 3) + 2 * Hq * d * 2
        gbsv = vbytes / (usv * 1e-6) / 1e9
        out["shapes"][name + "_varlen"] = {"query_heads": Hq, "kv_heads": H, "T_max": T,
                                           "seq_tokens": [int(x) for x in seq_T], "d": d, "us": usv,
                                           "algorithmic_bytes": vbytes, "gbs": gbsv,
                                           "hbm_frac": gbsv / PEAK_HBM_GBS, "cache_copies": copies}
        del caches, q, o, ws
        torch.cuda.empty_cache()
    return out


def _median_us(torch, fn, iters, rounds=5):
    """Median over `rounds` of the mean microseconds per call of fn() over
    `iters` back-to-back calls (HIP events on the launch stream). Each round
    starts with an untimed call that the first event is queued behind, so the
    GPU is busy when timing starts and the host's latency to the first timed
    launch after a synchronization is not counted. 300 untimed calls first:
    the first passes over freshly written caches of >= 1 GB run about 15%
    slower (74-76 us against 63 for the multi-head shape in one probe, the
    same with the binding or the bare C call)."""
    for _ in range(300):
        fn()
    v = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fn()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        v.append(a.elapsed_time(b) * 1e3 / iters)
    v.sort()
    return v[len(v) // 2]


def _per_call_us(torch, fn, iters):
    """Mean microseconds per call of fn(i), i = 0 .. iters-1: HIP events on the
    launch stream around `iters` back-to-back calls, after 3 untimed ones."""
    for i in range(3):
        fn(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(iters):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / iters


def _graph_per_call_us(torch, fn, reps, check):
    """Mean microseconds per call of fn(i), i = 0 .. reps-1, captured once in a
    HIP graph and replayed (no host launch cost per call). `check()` runs after
    every replay, with the eager work and synchronization in between, and must
    return True (the replay reproduced the eager result); None if it does not."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        if not check():
            return None
        times.append(a.elapsed_time(b) * 1e3 / reps)
    del g
    return float(np.median(times))


def decode_sweep(torch, comet, synth, iters=60):
    """The LLaMA-70B decode sweep (M in {1, 4, 16, 64}, K = 8192, N in {10240,
    8192, 28672}) on the INT4 layout: comet_w4ax_gemm, comet_quant_act and the
    pair, each timed over `iters` back-to-back calls that rotate through weight
    copies of >= 1 GB (the 256 MB last-level cache cannot serve them). HBM
    fraction of the GEMM from its algorithmic bytes (weight codes, scales and
    sums, activation codes and scales, fp16 Y) against 8 TB/s."""
    out = {"timing": f"HIP events around {iters} back-to-back calls per figure, weights rotated "
                     f"over copies of >= 1 GB; the *_graph_us figures replay the same {iters} calls from "
                     f"one captured HIP graph (no host launch cost; every replay checked against the "
                     f"eager result, null if one differed)", "shapes": {}}
    for N in (10240, 8192, 28672):
        cfg1 = synth.CONFIGS[f"decode_70b_n{N}_m1"]
        K, nb8 = cfg1.K, cfg1.nb8
        pk = comet.comet_pack_weights(synth.make_w(cfg1), synth.make_scores(cfg1), nb8)
        w0 = comet.upload_weights(pk)
        copies = copies_for(cfg1)
        ws = [w0] + [{k: (v.clone() if hasattr(v, "clone") else v) for k, v in w0.items()}
                     for _ in range(copies - 1)]
        for m in (1, 4, 16, 64):
            cfg = synth.CONFIGS[f"decode_70b_n{N}_m{m}"]
            X = torch.from_numpy(synth.make_x(cfg).view(np.float16)).cuda()
            Xq, xs = comet.comet_quant_act(X, w0["perm"], nb8)
            Y = torch.empty((m, N), dtype=torch.float16, device="cuda")
            g = _per_call_us(torch, lambda i: comet.comet_w4ax_gemm(Xq, xs, ws[i % copies], m, Y=Y), iters)
            q = _per_call_us(torch, lambda i: comet.comet_quant_act(X, ws[i % copies]["perm"], nb8, Xq=Xq,
                                                                    x_scale=xs), iters)

            def pair(i):
                w = ws[i % copies]
                comet.comet_quant_act(X, w["perm"], nb8, Xq=Xq, x_scale=xs)
                comet.comet_w4ax_gemm(Xq, xs, w, m, Y=Y)

            pq = _per_call_us(torch, pair, iters)
            # the same calls from a captured HIP graph: the kernels' own rate,
            # without the Python binding's launch cost per call
            pair(0)
            torch.cuda.synchronize()
            Y_ref, Xq_ref, xs_ref = Y.clone(), Xq.clone(), xs.clone()

            def same():
                return bool(torch.equal(Y, Y_ref) and torch.equal(Xq, Xq_ref) and torch.equal(xs, xs_ref))

            qg = _graph_per_call_us(torch, lambda i: comet.comet_quant_act(X, ws[i % copies]["perm"], nb8, Xq=Xq,
                                                                           x_scale=xs), iters, same)
            pg = _graph_per_call_us(torch, pair, iters, same)
            nbytes = gemm_bytes(m, N, K, nb8, "int4")
            gbs = nbytes / (g * 1e-6) / 1e9
            out["shapes"][f"m{m}_n{N}"] = {
                "M": m, "N": N, "K": K, "int8_blocks": nb8, "gemm_us": g, "quant_us": q, "pair_us": pq,
                "quant_graph_us": qg, "pair_graph_us": pg,
                "gemm_bytes": nbytes, "gemm_gbs": gbs, "gemm_hbm_frac": gbs / PEAK_HBM_GBS,
                "gemm_tops": 2.0 * m * N * K / (g * 1e-6) / 1e12, "weight_copies": copies}
            log(f"[bench] decode m={m} n={N}: gemm {g:.1f} us ({gbs:.0f} GB/s, "
                f"{gbs / PEAK_HBM_GBS:.2f} of HBM), quant {q:.1f} us, pair {pq:.1f} us; from a graph: "
                f"quant {qg if qg is None else round(qg, 1)} us, pair {pg if pg is None else round(pg, 1)} us")
        del ws, w0
        torch.cuda.empty_cache()
    return out


def layer_configs(torch, comet, synth, iters=50):
    """LLaMA-7B layers: q_proj (128 tokens; HBM binds: op/B below the ridge)
    and the MLP pair up/gate + down (1024 tokens; the matrix unit binds), on
    the FP6 layout with the split-K work queue where a grid is below one wave.
    GEMM and quantizer each over `iters` back-to-back calls, weights rotated
    over copies of >= 1 GB. Fractions against the instruction-mix peak (FP6
    for 4-bit blocks, INT8 for 8-bit ones), the dense INT8 peak, and HBM."""
    res = {"timing": f"HIP events around {iters} back-to-back calls per figure, weights rotated over "
                     f"copies of >= 1 GB"}
    for group, names in (("q_proj_7b", ["q_proj_7b"]), ("mlp_7b", ["up_gate_7b", "down_7b"])):
        g_out = {"layers": {}}
        tot_ops = tot_us = 0.0
        for name in names:
            l = Layer(name, copies_for(synth.CONFIGS[name]), torch, comet, synth)
            l.quant(l.w[0])
            gu = _per_call_us(torch, lambda i: l.gemm(l.w[i % len(l.w)]), iters)
            qu = _per_call_us(torch, lambda i: l.quant(l.w[i % len(l.w)]), iters)
            tops = l.ops / (gu * 1e-6) / 1e12
            gbs = l.gbytes / (gu * 1e-6) / 1e9
            bound = "hbm" if l.gbytes / (PEAK_HBM_GBS * 1e9) > l.ops / (l.peak * 1e12) else "mfma"
            g_out["layers"][name] = {
                "M": l.cfg.M, "N": l.cfg.N, "K": l.cfg.K, "int8_blocks": l.cfg.nb8, "gemm_us": gu,
                "quant_us": qu, "gemm_tops": tops, "gemm_gbs": gbs, "bound": bound,
                "frac_vs_mix_peak": tops / l.peak, "frac_vs_int8_peak": tops / PEAK_INT8_TOPS,
                "hbm_frac": gbs / PEAK_HBM_GBS, "mix_peak_tops": l.peak,
                "workspace_bytes": l.ws_bytes, "weight_copies": len(l.w)}
            log(f"[bench] {name}: gemm {gu:.1f} us ({tops:.0f} TOPS, {tops / l.peak:.3f} of the mix peak, "
                f"{gbs:.0f} GB/s), quant {qu:.1f} us")
            tot_ops += l.ops
            tot_us += gu
            del l
            torch.cuda.empty_cache()
        g_out["gemm_us"] = tot_us
        g_out["gemm_tops"] = tot_ops / (tot_us * 1e-6) / 1e12
        res[group] = g_out
    return res


def cpu_single_core(budget_s=12.0):
    """The oracle on one core for the small configurations: a bounded sample of
    rows of tiny, q_proj_7b, up_gate_7b, down_7b and the decode layers (M = 1),
    steps 3-5 (activation quantization, block partials, epilogue) with the
    weights quantized beforehand."""
    from gen import synth
    from oracle import oracle as O
    O.build(force=False)
    before = O.threads()
    O.set_threads(1)
    names = ["tiny", "q_proj_7b", "up_gate_7b", "down_7b"] + [f"decode_70b_n{n}_m1" for n in (10240, 8192, 28672)]
    per = budget_s / len(names)
    out = {}
    try:
        for name in names:
            cfg = synth.CONFIGS[name]
            X, W, score = synth.make_x(cfg, rows=min(cfg.M, 64)), synth.make_w(cfg), synth.make_scores(cfg)
            perm, flags = O.channel_order(score, cfg.nb8)
            qw, sw16, _ = O.quantize_weights(W, perm)
            rows, spent = 0, 0.0
            while rows < X.shape[0] and spent < per:
                t = time.perf_counter()
                O.forward_rows(X, perm, flags, qw, sw16, (rows, rows + 1))
                spent += time.perf_counter() - t
                rows += 1
            out[name] = {"rows": rows, "of_rows": cfg.M, "seconds": spent,
                         "tops": 2.0 * rows * cfg.N * cfg.K / spent / 1e12}
    finally:
        O.set_threads(before)
    return out


def cpu_baseline(layers, budget_s):
    """The oracle as it stands, on a bounded sample of rows of every layer: host
    time of steps 3-5 (activation quantization, block partials, epilogue) with
    the weights quantized beforehand, like the GPU path."""
    from oracle import oracle as O
    O.build(force=False)
    done_ops, spent, desc = 0.0, 0.0, []
    prep = []
    for l in layers:
        perm, flags = O.channel_order(l.host["score"], l.cfg.nb8)
        qw, sw16, _ = O.quantize_weights(l.host["W"], perm)
        prep.append((l, perm, flags, qw, sw16))
    per_layer = budget_s / len(layers)
    for l, perm, flags, qw, sw16 in prep:
        M, N, K = l.cfg.M, l.cfg.N, l.cfg.K
        rows, t_layer, chunk = 0, 0.0, 4
        while rows < M and t_layer < per_layer:
            c = min(chunk, M - rows)
            t = time.perf_counter()
            O.forward_rows(l.host["X"], perm, flags, qw, sw16, (rows, rows + c))
            dt = time.perf_counter() - t
            t_layer += dt
            rows += c
            done_ops += 2.0 * c * N * K
            if dt < 1.0:
                chunk = min(chunk * 2, 256)
        spent += t_layer
        desc.append(f"{l.name}: rows 0..{rows - 1} of {M}")
    return {"value": done_ops / spent / 1e12, "unit": "TOPS", "cores": O.threads(),
            "kind": "oracle", "sample": "; ".join(desc) + f" ({spent:.1f} s of host time)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_70b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fusion", action="store_true",
                    help="skip the fused-quantizer and asymmetric-variant ablations (outside the timed step)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kv4-only", action="store_true",
                    help="only the KV4 decode attention measurement (its JSON object), for profiling")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode sweep and the LLaMA-7B layers (outside the timed step)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the decode sweep and the LLaMA-7B layers (their JSON objects), for profiling")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import w4ax_mixed_precision_amd as comet
    from gen import synth
    comet.lib()
    assert torch.cuda.is_available(), "bench needs a GPU"
    if args.kv4_only:
        print(json.dumps({"kv4_decode_attention": kv4_attention_measure(torch, comet, synth)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"decode_70b": decode_sweep(torch, comet, synth),
                          "llama7b_layers": layer_configs(torch, comet, synth)}), flush=True)
        return

    layers = [Layer(n, copies_for(synth.CONFIGS[n]), torch, comet, synth)
              for n in WORKLOADS[args.workload]]
    step_ms, per = run_gpu(layers, args.steps, args.warmup, torch, comet)
    ops = sum(l.ops for l in layers)
    value = ops / (step_ms * 1e-3) / 1e12

    gemm_ms = sum(per[l.name]["gemm_ms"] for l in layers)
    gemm_ops = sum(l.ops for l in layers)
    gemm_bytes_total = sum(l.gbytes for l in layers)
    achieved_tops = gemm_ops / (gemm_ms * 1e-3) / 1e12
    achieved_gbs = gemm_bytes_total / (gemm_ms * 1e-3) / 1e9
    t_mfma = sum(l.ops / (l.peak * 1e12) for l in layers)
    peak_tops = gemm_ops / t_mfma / 1e12
    t_hbm = gemm_bytes_total / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": achieved_tops, "peak": peak_tops,
                "unit": "TFLOP/s", "frac": achieved_tops / peak_tops,
                "frac_vs_mix_peak": achieved_tops / peak_tops,
                "frac_vs_int8_peak": achieved_tops / PEAK_INT8_TOPS,
                "peak_basis": "dense MFMA peak of the instruction mix: FP6 10.1 POPS for 4-bit "
                              "blocks, INT8 5.0 POPS for 8-bit blocks (and for every block on "
                              "the INT4 layout); frac_vs_int8_peak is against the dense INT8 "
                              "peak (5.0 POPS) alone"}
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS}
    traffic, traffic_src = measured_traffic(args.workload)
    roof["traffic"] = traffic
    roof["traffic_source"] = traffic_src
    roof["algorithmic_bytes"] = gemm_bytes_total
    roof["kernel"] = "comet_w4ax_gemm"

    kernels = {}
    for l in layers:
        p = per[l.name]
        kernels[l.name] = {
            "gemm_us": p["gemm_ms"] * 1e3, "gemm_us_p10": p["gemm_ms_p10"] * 1e3,
            "gemm_us_p90": p["gemm_ms_p90"] * 1e3,
            "gemm_tops": l.ops / (p["gemm_ms"] * 1e-3) / 1e12,
            "gemm_frac_peak": l.ops / (p["gemm_ms"] * 1e-3) / 1e12 / l.peak,
            "gemm_gbs": l.gbytes / (p["gemm_ms"] * 1e-3) / 1e9,
            "quant_us": p["quant_ms"] * 1e3,
            "quant_gbs": l.qbytes / (p["quant_ms"] * 1e-3) / 1e9,
            "layout": l.layout, "gemm_peak_tops": l.peak,
            "weight_copies": len(l.w)}

    ablate = args.workload == "prefill_70b" and not args.no_fusion
    fusion = fusion_ablation(torch, comet, synth) if ablate else None
    swi = swiglu_ablation(torch, comet, synth) if ablate else None
    asym = asym_ablation(torch, comet, synth) if ablate else None
    qoq = qoq_ablation(torch, comet, synth) if ablate else None
    quik = quik_ablation(torch, comet, synth) if ablate else None
    kv4 = kv4_attention_measure(torch, comet, synth) if ablate else None

    configs = None
    if args.workload == "prefill_70b" and not args.no_configs:
        configs = {"decode_70b": decode_sweep(torch, comet, synth),
                   "llama7b_layers": layer_configs(torch, comet, synth)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(layers, args.cpu_seconds)
        if args.workload == "prefill_70b":
            cpu["single_core"] = cpu_single_core()

    out = {
        "metric": "W4Ax GEMM effective TOPS + % INT8-MFMA/HBM roofline, LLaMA-70B layer shapes",
        "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8+fp6(e2m3 exact int4 codes)",
        "data": "synthetic (seeded LLaMA-shaped activations with planted outlier channels, "
                "N(0,0.02) weights)",
        "config": {"workload": args.workload,
                   "layers": [{"name": l.name, "M": l.cfg.M, "K": l.cfg.K, "N": l.cfg.N,
                               "int8_blocks": l.cfg.nb8, "blocks": l.cfg.nb} for l in layers],
                   "step": "comet_quant_act + comet_w4ax_gemm per layer (the *_fp6 pair on "
                           "the FP6 layout when M > 64)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "norm_quant_fusion": fusion,
        "swiglu_quant_fusion": swi,
        "asym_activation_variant": asym,
        "qoq_w4a8_variant": qoq,
        "quik_fp16_outlier_variant": quik,
        "kv4_decode_attention": kv4,
        "configs": configs,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
