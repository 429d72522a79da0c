"""Per-layer SparseGPT solve time on one MI355X.

One step = the whole hot path for one linear layer with its calibration
activations already resident in HBM: zero H, H += X^T X over all tokens,
factor (H + lambda I)^{-1} -> U, prune W (mask selection, OBS compensation,
lazy updates).  Default workload: the 4096 x 4096 attention-projection layer
(bf16 W and X, 262,144 calibration tokens, 50% unstructured, block 128).

Prints ONE JSON line.  ``value`` is the per-layer wall time in seconds (lower
is better); per-phase times, algorithmic TFLOP/s, the roofline of the dominant
kernel (the Hessian) and the oracle's CPU time on a bounded sample ride along.
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


def algorithmic_work(m, n, N, B):
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


def cpu_baseline(cfg, pattern, W_host, X_host_sample, n_tok_total, rows_sample, bits=0):
    """The oracle as it stands, timed on host cores on a bounded sample of the
    same layer, scaled to one whole layer: Hessian on a token sample (scaled by
    tokens), the full n x n factor, the column sweep on a row sample (scaled
    by rows)."""
    m_rows = W_host.shape[0]
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    xs = X_host_sample.double().numpy()
    t0 = time.perf_counter()
    Hs = oracle.hessian([xs])
    t_h = time.perf_counter() - t0
    H_est = Hs * (n_tok_total / xs.shape[0])
    t0 = time.perf_counter()
    Hd, _ = oracle.dampen(H_est, cfg.damp)
    U = oracle.inverse_upper_factor(Hd)
    t_u = time.perf_counter() - t0
    Ws = W_host[:rows_sample].double().numpy()
    t0 = time.perf_counter()
    if bits:
        oracle.prune_quantized(Ws, U, pattern, cfg.blocksize, bits)
    else:
        oracle.prune(Ws, U, pattern, cfg.blocksize)
    t_p = time.perf_counter() - t0
    total = t_h * (n_tok_total / xs.shape[0]) + t_u + t_p * (m_rows / rows_sample)
    return {
        "value": total,
        "unit": "s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"Hessian on {xs.shape[0]} of {n_tok_total} tokens (x{n_tok_total // xs.shape[0]}), "
                   f"full {cfg.n}x{cfg.n} fp64 factor, sweep on {rows_sample} of {m_rows} rows "
                   f"(x{m_rows // rows_sample}); measured {t_h:.2f}+{t_u:.2f}+{t_p:.2f} s"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="attn_4096")
    ap.add_argument("--pattern", default=None)
    ap.add_argument("--shared", type=int, default=1,
                    help="prune this many matrices of the layer's shape that share its input "
                         "(stacked, one call with the shared factor)")
    ap.add_argument("--vec", type=int, default=1,
                    help="16: remove the chosen weights of each 16-column range together")
    ap.add_argument("--bits", type=int, default=0,
                    help="also round the kept weights to a per-row grid of 2^bits levels in the sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this size (for counter scaling)")
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
    cfg = synth.CONFIGS[args.config]
    pattern = args.pattern or cfg.patterns[0]
    m, n, N, B = cfg.m, cfg.n, cfg.tokens, cfg.blocksize
    print(f"[bench] generating {args.config}: W {m}x{n}, X {N}x{n} ({cfg.dtype})", file=sys.stderr,
          flush=True)
    if args.shared > 1:
        import dataclasses
        W = torch.cat([synth.make_weight(dataclasses.replace(cfg, config_id=cfg.config_id + 500 + i), dev)
                       for i in range(args.shared)])
        m = W.shape[0]
    else:
        W = synth.make_weight(cfg, dev)
    splits = [i * cfg.m for i in range(args.shared + 1)]
    X = synth.make_x(cfg, dev)
    torch.cuda.synchronize()

    H = torch.zeros(n, n, dtype=torch.float32, device=dev)
    Hinv = torch.empty(n, n, dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    W_out = torch.empty(m, n, dtype=torch.float32, device=dev)
    mask = torch.empty(m, n, dtype=torch.uint8, device=dev)
    ws_h = torch.empty(max(1, sg.sg_workspace_bytes(sg.SG_OP_HESSIAN, 0, n, N, 0)), dtype=torch.uint8,
                       device=dev)
    ws_f = torch.empty(sg.sg_workspace_bytes(sg.SG_OP_PREPARE_HINV, 0, n, 0, 0), dtype=torch.uint8,
                       device=dev)
    ws_p = torch.empty(sg.sg_workspace_bytes(sg.SG_OP_PRUNE, m, n, 0, B), dtype=torch.uint8, device=dev)
    codes = torch.empty(m, n, dtype=torch.uint8, device=dev) if args.bits else None

    def prune():
        if args.shared > 1:
            sg.sg_prune_layers_shared(W, splits, Hinv, pattern, B, bits=args.bits, W_out=W_out,
                                      mask_out=mask, codes_out=codes, workspace=ws_p)
        elif args.vec != 1:
            sg.sg_prune_layer_vector(W, Hinv, pattern, args.vec, B, W_out=W_out, mask_out=mask,
                                     workspace=ws_p)
        elif args.bits:
            sg.sg_prune_quantize_layer(W, Hinv, pattern, args.bits, B, W_out=W_out, mask_out=mask,
                                       codes_out=codes, workspace=ws_p)
        else:
            sg.sg_prune_layer(W, Hinv, pattern, B, W_out=W_out, mask_out=mask, workspace=ws_p)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        if marks is not None:
            marks[0].record()
        H.zero_()
        sg.sg_hessian_accumulate(H, X, workspace=ws_h)
        if marks is not None:
            marks[1].record()
        sg.sg_prepare_hinv(H, cfg.damp, Hinv=Hinv, info=info, workspace=ws_f)
        if marks is not None:
            marks[2].record()
        prune()
        if marks is not None:
            marks[3].record()

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    if int(info.item()) != 0:
        raise RuntimeError(f"factorisation failed: info={int(info.item())}")

    phase_marks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    hess_marks = [[ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start, t_end = ev(), ev()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        mk = phase_marks[i]
        mk[0].record()
        H.zero_()
        hess_marks[i][0].record()
        sg.sg_hessian_accumulate(H, X, workspace=ws_h)
        hess_marks[i][1].record()
        mk[1].record()
        sg.sg_prepare_hinv(H, cfg.damp, Hinv=Hinv, info=info, workspace=ws_f)
        mk[2].record()
        prune()
        mk[3].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (host wall {wall:.2f} s)",
          file=sys.stderr, flush=True)

    ph = {"hessian": 0.0, "factor": 0.0, "prune": 0.0}
    for mk in phase_marks:
        ph["hessian"] += mk[0].elapsed_time(mk[1])
        ph["factor"] += mk[1].elapsed_time(mk[2])
        ph["prune"] += mk[2].elapsed_time(mk[3])
    ph = {k: v / args.steps for k, v in ph.items()}
    t_hess_kernel_ms = sum(a.elapsed_time(b) for a, b in hess_marks) / args.steps

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

    export = None
    if pattern == "2:4":
        # 2:4 compressed export of the step's result (not part of the step):
        # HBM-bound, algorithmic bytes per weight 4 + 1 in, value bytes / 2 +
        # 1/8 out
        export = {}
        for vdt, vb in ((torch.float32, 4), (torch.bfloat16, 2)):
            vals = torch.empty(m, n // 2, dtype=vdt, device=dev)
            meta = torch.empty(m, (n + 7) // 8, dtype=torch.uint8, device=dev)
            for _ in range(2):
                sg.sg_pack_two_four(W_out, mask, value_dtype=vdt, values=vals, meta=meta)
            reps = 20
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                sg.sg_pack_two_four(W_out, mask, value_dtype=vdt, values=vals, meta=meta)
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
        tok_sample = min(N, 8192)
        rows = min(m, 256)
        cpu = cpu_baseline(cfg, pattern, W.cpu(), X[:tok_sample].cpu(), N, rows, args.bits)

    line = {
        "metric": "per-layer prune wall-time (s) + TFLOP/s & % MFMA/HBM roofline, 4096² → 28672×8192",
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
        "phase_roofline": {
            "hessian_frac_bf16": work["hessian"] / (ph["hessian"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "factor_frac_fp32": work["factor"] / (ph["factor"] * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
            "prune_tflops": (work["lazy"] + work["inblock"]) / (ph["prune"] * 1e-3) / 1e12,
        },
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
    if export is not None:
        line["two_four_export"] = export
    if args.shared > 1:
        line["matrices_per_s"] = args.shared / (ms * 1e-3)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
