"""Per-layer SparseGPT solve time on one MI355X.

One step = the whole hot path for one linear layer with its calibration
activations already resident in HBM: zero H, H += X^T X over all tokens,
factor (H + lambda I)^{-1} -> U, prune W (mask selection, OBS compensation,
lazy updates).  Default workload: the 8192 x 28672 down-projection layer
(bf16 W and X, 524,288 calibration tokens, 50% unstructured, block 128), the
largest of the layer shapes; the 4096- and 11008-wide layers are timed in the
same run after it (key "configs"), and four 4096 x 4096 layers with their own
inputs, factored and pruned together and one after another (key "layers").

Prints ONE JSON line.  ``value`` is the per-layer wall time in seconds (lower
is better).  Along with it: per-phase times, algorithmic TFLOP/s, each
phase's fraction of its roofline (the sweep and lazy-update kernels timed by
the profiler's kernel records over one extra prune call), the roofline of the
dominant kernel (the Hessian, timed with HIP events around its launch) and
the oracle's CPU time on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

METRIC = "per-layer prune wall-time (s) + TFLOP/s & % MFMA/HBM roofline, 4096² → 28672×8192"

# the other layer shapes, timed after the headline workload (name, pattern)
EXTRA = [("attn_4096", "0.5"), ("mlp_up_11008", "2:4"), ("mlp_down_11008", "0.6"),
         ("mlp_down_11008", "4:8"), ("mlp_down_28672", "2:4")]


def algorithmic_work(m, n, N, B):
    """Algorithmic flops (and the sweep's bytes) of one layer: H n(n+1)N,
    factor 2n^3/3, lazy sum 2 m w (n - i2), in-block sum m w (w - 1), sweep
    13 bytes per weight (W in, W_hat, errors, mask out)."""
    hess = n * (n + 1) * N
    factor = 2.0 * n ** 3 / 3.0
    lazy = 0.0
    inblock = 0.0
    for i1 in range(0, n, B):
        w = min(B, n - i1)
        lazy += 2.0 * m * w * (n - i1 - w)
        inblock += m * w * (w - 1)
    return {"hessian": float(hess), "factor": factor, "lazy": lazy, "inblock": inblock,
            "sweep_bytes": 13.0 * m * n}


def hessian_source_hash():
    h = hashlib.sha256()
    for f in ("hessian.hip", "hessian.h"):
        with open(os.path.join(ROOT, "post_pruning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per Hessian launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "hessian_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(workload)
    if not e or e.get("source_hash") != hessian_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(cfg, pattern, W_host, X_host_sample, n_tok_total, rows_sample, n_factor, bits=0):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same layer and scaled to one whole layer: the Hessian on a token
    sample (scaled by tokens), the factor at a smaller n (scaled by n^3), the
    column sweep on a row sample (scaled by rows)."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    m_rows, n = W_host.shape
    xs = X_host_sample.double().numpy()
    t0 = time.perf_counter()
    Hs = oracle.hessian([xs])
    t_h = time.perf_counter() - t0
    H_est = Hs * (n_tok_total / xs.shape[0])
    # the factor on the leading n_factor channels (same distribution)
    n_factor = min(n, n_factor)
    t0 = time.perf_counter()
    Hd_f, _ = oracle.dampen(H_est[:n_factor, :n_factor], cfg.damp)
    U = oracle.inverse_upper_factor(Hd_f)
    t_u = time.perf_counter() - t0
    if n > n_factor:
        # the sweep needs a factor of the full width: the diagonal one of the
        # damped diagonal (the sweep's cost does not depend on U's values)
        d = np.diag(H_est)
        U = np.diag(1.0 / np.sqrt(d + cfg.damp * d.mean()))
    Ws = W_host[:rows_sample].double().numpy()
    t0 = time.perf_counter()
    if bits:
        oracle.prune_quantized(Ws, U, pattern, cfg.blocksize, bits)
    else:
        oracle.prune(Ws, U, pattern, cfg.blocksize)
    t_p = time.perf_counter() - t0
    f_h = n_tok_total / xs.shape[0]
    f_u = (n / n_factor) ** 3
    f_p = m_rows / rows_sample
    total = t_h * f_h + t_u * f_u + t_p * f_p
    return {
        "value": total,
        "unit": "s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"Hessian on {xs.shape[0]} of {n_tok_total} tokens (x{f_h:.0f}), fp64 factor at "
                   f"n = {n_factor} (x{f_u:.1f} = (n/{n_factor})^3), sweep on {rows_sample} of {m_rows} "
                   f"rows (x{f_p:.0f}); measured {t_h:.2f} + {t_u:.2f} + {t_p:.2f} s on "
                   f"{cores} cores (sched_getaffinity)"),
    }


def kernel_attribution(fn):
    """Device time per kernel over one call of fn, from the profiler's kernel
    records: {kernel name: (calls, total ms)}."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    out = {}
    for e in prof.key_averages():
        t = getattr(e, "device_time_total", None)
        if t is None:
            t = getattr(e, "cuda_time_total", 0.0)
        if t and t > 0:
            out[e.key] = (int(e.count), t / 1e3)
    return out


def _short(name):
    """'void sg::(anonymous namespace)::sweep_kernel<0, 0>(float*, ...)' ->
    'sweep_kernel<0, 0>'."""
    s = name.replace("(anonymous namespace)::", "")
    s = s.split("(")[0].strip()
    if s.startswith("void "):
        s = s[5:]
    head = s.split("<")[0]
    if "::" in head:
        s = s[len(head.rsplit("::", 1)[0]) + 2:]
    return s


def _sum_kernels(attr, base):
    calls, ms = 0, 0.0
    for k, (c, t) in attr.items():
        if _short(k).split("<")[0] == base:
            calls += c
            ms += t
    return calls, ms


class Layer:
    """Device buffers and one step of the path for one workload."""

    def __init__(self, sg, cfg, pattern, dev, args, X=None):
        import torch

        import synth
        self.sg, self.cfg, self.pattern, self.args = sg, cfg, pattern, args
        m, n, N, B = cfg.m, cfg.n, cfg.tokens, cfg.blocksize
        if args.shared > 1:
            import dataclasses
            W = torch.cat([synth.make_weight(dataclasses.replace(cfg, config_id=cfg.config_id + 500 + i), dev)
                           for i in range(args.shared)])
            m = W.shape[0]
        else:
            W = synth.make_weight(cfg, dev)
        self.W = W
        self.m, self.n, self.N, self.B = m, n, N, B
        self.splits = [i * cfg.m for i in range(args.shared + 1)]
        self.X = X if X is not None else synth.make_x(cfg, dev)
        self.H = torch.zeros(n, n, dtype=torch.float32, device=dev)
        self.Hinv = torch.empty(n, n, dtype=torch.float32, device=dev)
        self.info = torch.zeros(1, dtype=torch.int32, device=dev)
        self.W_out = torch.empty(m, n, dtype=torch.float32, device=dev)
        self.mask = torch.empty(m, n, dtype=torch.uint8, device=dev)
        self.ws_h = torch.empty(max(1, sg.sg_workspace_bytes(sg.SG_OP_HESSIAN, 0, n, N, 0)),
                                dtype=torch.uint8, device=dev)
        self.ws_f = torch.empty(sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, n, 0, 0), dtype=torch.uint8,
                                device=dev)
        self.ws_p = torch.empty(sg.sg_workspace_bytes(sg.SG_OP_PRUNE, m, n, 0, B), dtype=torch.uint8,
                                device=dev)
        self.codes = torch.empty(m, n, dtype=torch.uint8, device=dev) if args.bits else None
        # the factor's update stream and events (used above n = 4096)
        self.side = torch.cuda.Stream(device=dev)

    def hessian(self):
        self.H.zero_()
        self.sg.sg_hessian_accumulate(self.H, self.X, workspace=self.ws_h)

    def factor(self):
        self.sg.sg_prepare_hinv(self.H, self.cfg.damp, Hinv=self.Hinv, info=self.info, workspace=self.ws_f,
                                update_stream=self.side)

    def prune(self):
        sg, a = self.sg, self.args
        if a.shared > 1:
            sg.sg_prune_layers_shared(self.W, self.splits, self.Hinv, self.pattern, self.B, bits=a.bits,
                                      W_out=self.W_out, mask_out=self.mask, codes_out=self.codes,
                                      workspace=self.ws_p)
        elif a.vec != 1:
            sg.sg_prune_layer_vector(self.W, self.Hinv, self.pattern, a.vec, self.B, W_out=self.W_out,
                                     mask_out=self.mask, workspace=self.ws_p)
        elif a.bits:
            sg.sg_prune_quantize_layer(self.W, self.Hinv, self.pattern, a.bits, self.B, W_out=self.W_out,
                                       mask_out=self.mask, codes_out=self.codes, workspace=self.ws_p)
        else:
            sg.sg_prune_layer(self.W, self.Hinv, self.pattern, self.B, W_out=self.W_out, mask_out=self.mask,
                              workspace=self.ws_p)

    def step(self):
        self.hessian()
        self.factor()
        self.prune()

    def timed(self, steps, warmup, label):
        """warmup + steps; returns (ms per step, phase ms, Hessian launch ms)."""
        import torch
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        for i in range(warmup):
            self.step()
            torch.cuda.synchronize()
            print(f"[bench] {label}: warmup {i + 1}/{warmup} done", file=sys.stderr, flush=True)
        if int(self.info.item()) != 0:
            raise RuntimeError(f"{label}: factorisation failed: info={int(self.info.item())}")
        marks = [[ev() for _ in range(5)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0, t1 = ev(), ev()
        t0.record()
        for i in range(steps):
            mk = marks[i]
            mk[0].record()
            self.H.zero_()
            mk[1].record()  # the Hessian launch alone, on the stream it runs on
            self.sg.sg_hessian_accumulate(self.H, self.X, workspace=self.ws_h)
            mk[2].record()
            self.factor()
            mk[3].record()
            self.prune()
            mk[4].record()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        ph = {"hessian": 0.0, "factor": 0.0, "prune": 0.0}
        hk = 0.0
        for mk in marks:
            ph["hessian"] += mk[0].elapsed_time(mk[2])
            hk += mk[1].elapsed_time(mk[2])
            ph["factor"] += mk[2].elapsed_time(mk[3])
            ph["prune"] += mk[3].elapsed_time(mk[4])
        ph = {k: v / steps for k, v in ph.items()}
        print(f"[bench] {label}: timed {steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
        return ms, ph, hk / steps

    def fractions(self, ph, attr=None):
        w = algorithmic_work(self.m, self.n, self.N, self.B)
        out = {
            "hessian_frac_bf16": w["hessian"] / (ph["hessian"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "factor_frac_fp32": w["factor"] / (ph["factor"] * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "prune_tflops": (w["lazy"] + w["inblock"]) / (ph["prune"] * 1e-3) / 1e12,
        }
        if attr:
            c_s, t_s = _sum_kernels(attr, "sweep_kernel")
            c_l, t_l = _sum_kernels(attr, "lazy_kernel")
            c_q, t_q = _sum_kernels(attr, "select_pass_kernel")
            if t_s > 0:
                out["sweep_hbm_frac"] = w["sweep_bytes"] / (t_s * 1e-3) / 1e9 / PEAK_HBM_GBS
                out["sweep_kernels_ms"] = t_s
                out["sweep_launches"] = c_s
            if t_l > 0:
                out["lazy_frac_fp32"] = w["lazy"] / (t_l * 1e-3) / 1e12 / PEAK_FP32_TFLOPS
                out["lazy_kernels_ms"] = t_l
            if t_q > 0:
                out["select_kernels_ms"] = t_q
        return out


def measure_peaks(dev):
    """The machine peaks the roofline fractions are quoted against, measured:
    MFMA chains on register operands (bf16 16x16x32 and fp32 16x16x4, eight
    waves per SIMD) and a 4 GiB device copy and read (libsg_peaks.so)."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "post_pruning_amd", "libsg_peaks.so"))
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timeit(call, reps=5):
        call()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            assert call() == 0
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    blocks, iters = 2048, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    waves = blocks * 4
    res = {}
    t = timeit(lambda: lib.sgp_mfma_bf16(iters, blocks, ctypes.c_void_p(out.data_ptr()), st))
    fl = waves * iters * 8 * 2.0 * 16 * 16 * 32
    res["mfma_bf16_tflops"] = fl / (t * 1e-3) / 1e12
    t = timeit(lambda: lib.sgp_mfma_f32(iters, blocks, ctypes.c_void_p(out.data_ptr()), st))
    fl = waves * iters * 8 * 2.0 * 16 * 16 * 4
    res["mfma_f32_tflops"] = fl / (t * 1e-3) / 1e12
    nbytes = 4 << 30
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    n4 = nbytes // 16
    cb = 256 * 16
    t = timeit(lambda: lib.sgp_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                    ctypes.c_int64(n4), cb, st))
    res["hbm_copy_gbs"] = 2.0 * nbytes / (t * 1e-3) / 1e9
    red = torch.empty(cb * 256, dtype=torch.float32, device=dev)
    t = timeit(lambda: lib.sgp_read(ctypes.c_void_p(a.data_ptr()), ctypes.c_int64(n4), cb,
                                    ctypes.c_void_p(red.data_ptr()), st))
    res["hbm_read_gbs"] = nbytes / (t * 1e-3) / 1e9
    res["datasheet"] = {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "mfma_f32_tflops": PEAK_FP32_TFLOPS,
                        "hbm_gbs": PEAK_HBM_GBS}
    res["probe"] = (f"{blocks} workgroups x 4 waves x {iters} rounds of 8 independent MFMAs; "
                    f"4 GiB float4 copy / read over {cb} workgroups; mean of 5 launches after one warm-up")
    return res


def bench_layers(sg, K, args, dev):
    """K layers of the 4096 x 4096 attention-projection shape, each with its
    own weights and calibration activations.  Sequential: per layer Hessian,
    factor, prune.  Batched: per layer Hessian and factor, then one
    sg_prune_layers_batched over the K stacked matrices with their own
    factors.  Overlapped: as batched, with each layer's factor on a second
    stream beside the next layer's Hessian (the factor's panel chain leaves
    most CUs idle).  Batched factor: per layer Hessian, then one
    sg_prepare_hinv_batched over the K Hessians and one batched prune.
    Returns ({form: ms per K layers, ...}, config, pattern)."""
    import dataclasses

    import torch

    import synth
    base = synth.CONFIGS["attn_4096"]
    pattern = args.pattern or base.patterns[0]
    cfgs = [dataclasses.replace(base, config_id=600 + i) for i in range(K)]
    Ls = []
    for i, c in enumerate(cfgs):
        print(f"[bench] generating layer {i + 1}/{K}", file=sys.stderr, flush=True)
        Ls.append(Layer(sg, c, pattern, dev, args))
    W_all = torch.cat([L.W for L in Ls])
    splits = [i * base.m for i in range(K + 1)]
    W_out = torch.empty(K * base.m, base.n, dtype=torch.float32, device=dev)
    mask = torch.empty(K * base.m, base.n, dtype=torch.uint8, device=dev)
    ws = torch.empty(sg.sg_workspace_bytes(sg.SG_OP_PRUNE, K * base.m, base.n, 0, base.blocksize),
                     dtype=torch.uint8, device=dev)
    Hinvs = [L.Hinv for L in Ls]
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def sequential():
        for L in Ls:
            L.step()

    def batched(marks=None):
        for L in Ls:
            L.hessian()
            L.factor()
        if marks is not None:
            marks.record()
        sg.sg_prune_layers_batched(W_all, splits, Hinvs, pattern, base.blocksize, W_out=W_out, mask_out=mask,
                                   workspace=ws)

    Hs = [L.H for L in Ls]
    infos = torch.zeros(K, dtype=torch.int32, device=dev)
    ws_fb = torch.empty(K * sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, base.n), dtype=torch.uint8,
                        device=dev)

    def factors_batched():
        sg.sg_prepare_hinv_batched(Hs, base.damp, Hinvs=Hinvs, info=infos, workspace=ws_fb)

    def batched_factor(marks=None):
        for L in Ls:
            L.hessian()
        factors_batched()
        if marks is not None:
            marks.record()
        sg.sg_prune_layers_batched(W_all, splits, Hinvs, pattern, base.blocksize, W_out=W_out, mask_out=mask,
                                   workspace=ws)

    fstream = torch.cuda.Stream(device=dev)  # default priority

    def overlapped(marks=None):
        main = torch.cuda.current_stream()
        for L in Ls:
            L.hessian()
            done = torch.cuda.Event()
            done.record(main)
            fstream.wait_event(done)
            with torch.cuda.stream(fstream):
                L.factor()
        main.wait_stream(fstream)
        if marks is not None:
            marks.record()
        sg.sg_prune_layers_batched(W_all, splits, Hinvs, pattern, base.blocksize, W_out=W_out, mask_out=mask,
                                   workspace=ws)

    res = {}
    for name, fn in (("sequential", sequential), ("batched", batched), ("overlapped", overlapped),
                     ("batched_factor", batched_factor)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = ev(), ev()
        pm = [ev() for _ in range(args.steps)]
        t0.record()
        for i in range(args.steps):
            if name != "sequential":
                fn(pm[i])
            else:
                fn()
        t1.record()
        torch.cuda.synchronize()
        res[name] = t0.elapsed_time(t1) / args.steps
        print(f"[bench] {K} layers {name}: {res[name]:.3f} ms/step", file=sys.stderr, flush=True)
    # the overlapped form computes the same factors and result, bit for bit
    batched()
    torch.cuda.synchronize()
    ref = (W_out.clone(), mask.clone(), [h.clone() for h in Hinvs])
    for name, fn in (("overlapped", overlapped), ("batched_factor", batched_factor)):
        fn()
        torch.cuda.synchronize()
        if not (torch.equal(W_out, ref[0]) and torch.equal(mask, ref[1]) and
                all(torch.equal(a, b) for a, b in zip(Hinvs, ref[2]))):
            raise RuntimeError(f"{name} layers differ from the batched form")
        if name == "batched_factor" and infos.tolist() != [0] * K:
            raise RuntimeError(f"batched factor info {infos.tolist()}")
    del ref
    # the factors alone: one batched call against one call per layer
    for name, fn in (("factors_batched_ms", factors_batched),
                     ("factors_sequential_ms", lambda: [L.factor() for L in Ls])):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    # the batched prune alone
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        sg.sg_prune_layers_batched(W_all, splits, Hinvs, pattern, base.blocksize, W_out=W_out, mask_out=mask,
                                   workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    res["batched_prune_ms"] = e0.elapsed_time(e1) / args.steps
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(args.steps):
        for L in Ls:
            L.prune()
    e1.record()
    torch.cuda.synchronize()
    res["sequential_prune_ms"] = e0.elapsed_time(e1) / args.steps
    return res, base, pattern


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="mlp_down_28672")
    ap.add_argument("--pattern", default=None)
    ap.add_argument("--shared", type=int, default=1,
                    help="prune this many matrices of the layer's shape that share its input "
                         "(stacked, one call with the shared factor)")
    ap.add_argument("--vec", type=int, default=1,
                    help="16: remove the chosen weights of each 16-column range together")
    ap.add_argument("--bits", type=int, default=0,
                    help="also round the kept weights to a per-row grid of 2^bits levels in the sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip timing the other layer shapes")
    ap.add_argument("--no-attribution", action="store_true",
                    help="skip the profiler's per-kernel times (e.g. when run under rocprofv3)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this size (for counter scaling)")
    ap.add_argument("--layers", type=int, default=0,
                    help="K > 1: K attention-shaped layers with their own inputs, pruned sequentially "
                         "and in one batched call; reports layers/s")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the machine peaks (MFMA bf16/fp32, HBM copy/read) and print them")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this solver runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_pruning_amd as sg
    import synth

    sg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.peaks:
        print(json.dumps({"measured_peaks": measure_peaks(dev)}))
        return
    if args.layers > 1:
        K = args.layers
        res, base, pattern = bench_layers(sg, K, args, dev)
        forms = {
            "overlapped": "per layer Hessian and factor (each factor on a second stream beside the next "
                          "Hessian), one batched prune",
            "batched_factor": "per layer Hessian, one batched factor of the K Hessians, one batched prune",
        }
        best = min(forms, key=lambda f: res[f])
        ms = res[best]
        print(json.dumps({
            "metric": METRIC, "value": ms / K / 1e3, "unit": "s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 inputs, fp32 accumulate/solve",
            "data": "synthetic (seeded; shapes and distributions of the layer)",
            "config": {"workload": f"{K} x attn_4096 layers with their own inputs: W 4096x4096 bf16, "
                                   f"X 262144x4096 bf16 each, pattern {pattern}, blocksize {base.blocksize}; "
                                   f"{forms[best]}",
                       "layers": K, "pattern": pattern, "form": best},
            "layers_per_s": K / (ms * 1e-3),
            "batched_ms_per_step": res["batched"],
            "batched_layers_per_s": K / (res["batched"] * 1e-3),
            "sequential_ms_per_step": res["sequential"],
            "sequential_layers_per_s": K / (res["sequential"] * 1e-3),
            "overlapped_ms_per_step": res["overlapped"],
            "batched_factor_ms_per_step": res["batched_factor"],
            "batched_factor_layers_per_s": K / (res["batched_factor"] * 1e-3),
            "batched_prune_ms": res["batched_prune_ms"],
            "sequential_prune_ms": res["sequential_prune_ms"],
            "factors_batched_ms": res["factors_batched_ms"],
            "factors_sequential_ms": res["factors_sequential_ms"],
        }))
        return
    cfg = synth.CONFIGS[args.config]
    pattern = args.pattern or cfg.patterns[0]
    print(f"[bench] generating {args.config}: W {cfg.m}x{cfg.n}, X {cfg.tokens}x{cfg.n} ({cfg.dtype})",
          file=sys.stderr, flush=True)
    L = Layer(sg, cfg, pattern, dev, args)
    torch.cuda.synchronize()
    ms, ph, t_hess_kernel_ms = L.timed(args.steps, args.warmup, args.config)
    m, n, N, B = L.m, L.n, L.N, L.B

    attr = None
    if not args.no_attribution:
        try:
            attr = kernel_attribution(L.prune)
            f_attr = kernel_attribution(L.factor)
            attr_factor = {k: v for k, v in f_attr.items()}
        except Exception as e:  # the profiler is context, never the measurement
            print(f"[bench] kernel attribution unavailable: {e!r}", file=sys.stderr, flush=True)
            attr, attr_factor = None, None
    else:
        attr_factor = None
    fr = L.fractions(ph, attr)
    work = algorithmic_work(m, n, N, B)
    total_flops = work["hessian"] + work["factor"] + work["lazy"] + work["inblock"]
    achieved = work["hessian"] / (t_hess_kernel_ms * 1e-3) / 1e12
    traffic = load_traffic(args.config)

    if args.copy_calibration_mb > 0:
        nb = args.copy_calibration_mb * (1 << 20)
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    export = None
    if pattern == "2:4":
        # 2:4 compressed export of the step's result (not part of the step):
        # HBM-bound, algorithmic bytes per weight 4 + 1 in, value bytes / 2 +
        # 1/8 out
        export = {}
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        for vdt, vb in ((torch.float32, 4), (torch.bfloat16, 2)):
            vals = torch.empty(m, n // 2, dtype=vdt, device=dev)
            meta = torch.empty(m, (n + 7) // 8, dtype=torch.uint8, device=dev)
            for _ in range(2):
                sg.sg_pack_two_four(L.W_out, L.mask, value_dtype=vdt, values=vals, meta=meta)
            reps = 20
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                sg.sg_pack_two_four(L.W_out, L.mask, value_dtype=vdt, values=vals, meta=meta)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            nbytes = m * n * 5.0 + m * (n // 2) * vb + m * ((n + 7) // 8)
            gbs = nbytes / (t * 1e-3) / 1e9
            export["values_" + ("f32" if vb == 4 else "bf16")] = {
                "kernel": "pack24_kernel (sg_pack_two_four)", "bound": "hbm", "ms": t,
                "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "algorithmic_bytes": nbytes}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a host sample", file=sys.stderr, flush=True)
        tok_sample = min(N, 4096 if n > 8192 else 8192)
        rows = min(m, 16 if n > 8192 else 256)
        n_factor = min(n, 8192)
        cpu = cpu_baseline(cfg, pattern, L.W.cpu(), L.X[:tok_sample].cpu(), N, rows, n_factor, args.bits)

    main_key = f"{args.config} {pattern}"
    extra = {}
    if not args.no_extra and args.shared == 1 and args.vec == 1 and not args.bits:
        # free the headline layer's buffers, then time the other shapes
        keepX = L.X if args.config == "mlp_down_28672" else None
        del L
        torch.cuda.empty_cache()
        cache = {}
        for name, pat in EXTRA:
            key = f"{name} {pat}"
            if key == main_key:
                continue
            c = synth.CONFIGS[name]
            xsrc = c.x_source or name
            if name == "mlp_down_28672" and keepX is not None:
                X = keepX
            elif xsrc in cache:
                X = cache[xsrc]
            else:
                cache.clear()
                torch.cuda.empty_cache()
                X = synth.make_x(c, dev)
                cache[xsrc] = X
            Lx = Layer(sg, c, pat, dev, args, X=X)
            e_ms, e_ph, e_hk = Lx.timed(3, 1, key)
            e_attr = None
            if not args.no_attribution and attr is not None:
                try:
                    e_attr = kernel_attribution(Lx.prune)
                except Exception:
                    e_attr = None
            e_fr = Lx.fractions(e_ph, e_attr)
            w = algorithmic_work(Lx.m, Lx.n, Lx.N, Lx.B)
            extra[key] = {
                "ms": e_ms, "phases_ms": {k: round(v, 4) for k, v in e_ph.items()},
                "tflops_algorithmic": (w["hessian"] + w["factor"] + w["lazy"] + w["inblock"]) / (e_ms * 1e-3) / 1e12,
                "hessian_launch_ms": e_hk,
                "phase_roofline": e_fr,
            }
            del Lx
            torch.cuda.empty_cache()
        keepX = None
        cache.clear()
        # several layers with their own inputs (4 x attn_4096): one batched
        # factor and one batched prune against one layer after another
        la = argparse.Namespace(**{**vars(args), "steps": 3, "warmup": 1, "pattern": None})
        lres, lbase, lpat = bench_layers(sg, 4, la, dev)
        layers = {
            "workload": f"4 x attn_4096 layers with their own inputs, pattern {lpat}, blocksize {lbase.blocksize}",
            "sequential_layers_per_s": 4 / (lres["sequential"] * 1e-3),
            "batched_prune_layers_per_s": 4 / (lres["batched"] * 1e-3),
            "batched_factor_and_prune_layers_per_s": 4 / (lres["batched_factor"] * 1e-3),
            "factors_ms": {"batched": lres["factors_batched_ms"], "one_by_one": lres["factors_sequential_ms"]},
            "prune_ms": {"batched": lres["batched_prune_ms"], "one_by_one": lres["sequential_prune_ms"]},
        }
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": ms / 1e3,
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs, fp32 accumulate/solve" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and distributions of the layer)",
        "config": {
            "workload": f"{args.config}: W {m}x{n} {cfg.dtype}, X {N}x{n} {cfg.dtype}, "
                        f"pattern {pattern}, blocksize {B}, damp {cfg.damp}"
                        + (f", kept weights on a {args.bits}-bit grid" if args.bits else "")
                        + (f", chosen weights removed {args.vec} columns at a time" if args.vec != 1 else ""),
            "m": m, "n": n, "tokens": N, "pattern": pattern, "blocksize": B,
            "quant_bits": args.bits or None,
            "shared_matrices": args.shared,
            "joint_range": args.vec,
        },
        "phases_ms": {k: round(v, 4) for k, v in ph.items()},
        "tflops_algorithmic": total_flops / (ms * 1e-3) / 1e12,
        "phase_roofline": fr,
        "roofline": {
            "kernel": "hess_bf16_dma_kernel (sg_hessian_accumulate, one launch per step)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "launch_ms": t_hess_kernel_ms,
            "algorithmic_flops_per_launch": work["hessian"],
        },
        "cpu_baseline": cpu,
    }
    if attr:
        line["prune_kernels_ms"] = {_short(k): round(t, 4)
                                    for k, (c, t) in sorted(attr.items(), key=lambda kv: -kv[1][1])[:8]}
    if attr_factor:
        line["factor_kernels_ms"] = {_short(k): round(t, 4) for k, (c, t) in
                                     sorted(attr_factor.items(), key=lambda kv: -kv[1][1])[:6]}
    if extra:
        line["configs"] = extra
        line["layers"] = layers
    if export is not None:
        line["two_four_export"] = export
    if args.shared > 1:
        line["matrices_per_s"] = args.shared / (ms * 1e-3)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
