"""GPU parity of the joint sparse + quantized sweep (sg_prune_quantize_layer)
against the fp64 oracle (oracle.prune_quantized).

Same seeded inputs on both sides.  The GPU decides masks and grid codes in
fp32, the oracle in fp64, so decisions are compared as the pruning masks are:
  * grid (scale, zero) from the original rows: scale to 1e-6 relative, zero
    exact;
  * free run: exact per-block / per-group prune counts, per-row mask agreement
    >= 99.5%, and W_hat = scale * (code - zero) exactly in fp32, pruned
    entries +0.0, their codes the zero point;
  * along the GPU's own trajectory (oracle with the GPU's mask and codes
    forced): every selection consistent with the oracle's saliencies up to a
    relative gap TAU, every code the rounding of the oracle's value at that
    point except within TIE of a half-way point, and W_hat within 1e-4
    relative Frobenius;
  * reconstruction error of the GPU's W_hat against the free oracle's within
    1e-3 relative.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TAU = 1e-3
TIE = 1e-4

CASES = [
    # name, m, n, tokens, dtype, act, outliers, factor, (pattern, bits) list, blocksize
    ("attn_q", 256, 512, 16384, "bf16", "linear", 8, 20.0, (("0.5", 4), ("0.0", 8)), 128),
    ("mlpup_q", 384, 512, 8192, "bf16", "linear", 8, 20.0, (("2:4", 4), ("0.5/row", 3)), 128),
    ("ragged_q", 200, 1000, 3000, "bf16", "linear", 4, 20.0, (("0.5", 3),), 128),
    ("b32_q", 96, 256, 4096, "f32", "relu", 2, 10.0, (("16:32", 4), ("4:8", 2)), 32),
]


@pytest.fixture(autouse=True)
def _announce(request):
    sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


@pytest.fixture(scope="module")
def sg():
    import post_pruning_amd as sg
    sg.load_library()
    return sg


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _counts(mask, pattern, B):
    m, n = mask.shape
    if ":" in pattern:
        N, M = map(int, pattern.split(":"))
        assert np.all(mask.reshape(m, -1, M).sum(axis=2) == M - N)
    elif pattern.endswith("/row"):
        p = float(pattern[:-4])
        for j in range(0, n, B):
            w = min(B, n - j)
            assert np.all(mask[:, j:j + w].sum(axis=1) == math.floor(p * w))
    else:
        p = float(pattern)
        for j in range(0, n, B):
            w = min(B, n - j)
            assert int(mask[:, j:j + w].sum()) == math.floor(p * m * w)


def _selection_consistent(S, g, pattern, B):
    m, n = g.shape
    if ":" in pattern or pattern.endswith("/row"):
        M = int(pattern.split(":")[1]) if ":" in pattern else B
        for j in range(0, n, M):
            s, gg = S[:, j:j + M], g[:, j:j + M]
            hi = np.where(gg, s, -np.inf).max(axis=1)
            lo = np.where(~gg, s, np.inf).min(axis=1)
            assert not np.any(hi > lo * (1 + TAU) + 1e-300), f"group at column {j}"
    else:
        for j in range(0, n, B):
            s, gg = S[:, j:j + B], g[:, j:j + B]
            if gg.any() and (~gg).any():
                assert s[gg].max() <= s[~gg].min() * (1 + TAU) + 1e-300, f"block at column {j}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prune_quantize_parity(sg, case):
    name, m, n, tokens, dt, act, outl, fac, specs, B = case
    cfg = synth.LayerConfig(name, m, n, tokens, 0.02, dt, act, outl, fac,
                            tuple(p for p, _ in specs), B, config_id=950 + CASES.index(case),
                            chunk_tokens=tokens)
    W = synth.make_weight(cfg, "cpu")
    X = synth.make_x(cfg, "cpu")
    Wd = W.double().numpy()
    H = oracle.hessian([X.double().numpy()])
    Hd, _ = oracle.dampen(H, cfg.damp)
    U = oracle.inverse_upper_factor(Hd)
    Hg = torch.zeros(n, n, device="cuda")
    sg.sg_hessian_accumulate(Hg, X.cuda())
    Hinv, info = sg.sg_prepare_hinv(Hg, cfg.damp)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    Wc = W.cuda()
    for pattern, bits in specs:
        sys.stderr.write(f"[gpu-case] {name} pattern {pattern} bits {bits}\n")
        sys.stderr.flush()
        Wh, mask, codes, scale, zero = sg.sg_prune_quantize_layer(Wc, Hinv, pattern, bits, B)
        torch.cuda.synchronize()
        Whg = Wh.cpu().numpy()
        gm = mask.cpu().numpy().astype(bool)
        cg = codes.cpu().numpy()
        sc = scale.cpu().numpy()
        zr = zero.cpu().numpy()
        # grid
        so, zo = oracle.quant_grid(Wd, bits)
        assert np.abs(sc - so).max() <= 1e-6 * np.abs(so).max()
        assert np.array_equal(zr.astype(np.float64), zo)
        # structure of the GPU result
        _counts(gm, pattern, B)
        assert np.all(Whg[gm] == 0.0) and not np.any(np.signbit(Whg[gm]))
        assert np.all(cg[gm] == zr[np.nonzero(gm)[0]])
        deq = (sc[:, None] * (cg.astype(np.float32) - zr[:, None])).astype(np.float32)
        assert np.array_equal(np.where(gm, 0.0, deq), np.where(gm, 0.0, Whg))
        # free oracle
        Who, Mo, _, Co, _, _ = oracle.prune_quantized(Wd, U, pattern, B, bits)
        agree = (gm == Mo).mean(axis=1)
        assert agree.min() >= 0.995, f"min row mask agreement {agree.min():.5f}"
        code_agree = float((cg == Co).mean())
        sys.stderr.write(f"[gpu-case] code agreement with the free oracle {code_agree:.6f}\n")
        # along the GPU trajectory
        Whf, _, _, Cf, _, _, tr = oracle.prune_quantized(Wd, U, pattern, B, bits, mask_in=gm,
                                                         codes_in=cg, return_trace=True)
        _selection_consistent(tr["saliency"], gm, pattern, B)
        y = tr["at_quant"] / so[:, None]
        frac = np.abs(y - np.floor(y) - 0.5)
        want = oracle.quant_code(tr["at_quant"], so[:, None], zo[:, None], bits)
        bad = (~gm) & (cg != want) & (frac > TIE)
        assert not bad.any(), f"codes off the oracle's rounding at {np.argwhere(bad)[:5]}"
        assert _rel(Whg, Whf) <= 1e-4
        # reconstruction error against the free oracle
        E_g = oracle.reconstruction_error_from_hessian(Wd, Whg, H)
        E_o = oracle.reconstruction_error_from_hessian(Wd, Who, H)
        assert abs(E_g - E_o) <= 1e-3 * E_o, f"{E_g} vs {E_o}"
        # determinism
        Wh2, mask2, codes2, _, _ = sg.sg_prune_quantize_layer(Wc, Hinv, pattern, bits, B)
        assert torch.equal(Wh, Wh2) and torch.equal(mask, mask2) and torch.equal(codes, codes2)


def test_prune_quantize_forced_mask_matches_plain_prune_mask(sg):
    # a forced mask is taken as given; with 8 bits the result stays close to
    # pruning alone (same mask)
    case = CASES[0]
    name, m, n, tokens, dt, act, outl, fac, specs, B = case
    cfg = synth.LayerConfig(name, m, n, tokens, 0.02, dt, act, outl, fac, ("0.5",), B,
                            config_id=950, chunk_tokens=tokens)
    W = synth.make_weight(cfg, "cuda")
    X = synth.make_x(cfg, "cuda")
    Hg = torch.zeros(n, n, device="cuda")
    sg.sg_hessian_accumulate(Hg, X)
    Hinv, _ = sg.sg_prepare_hinv(Hg, cfg.damp)
    Wp, mp = sg.sg_prune_layer(W, Hinv, "0.5", B)
    Wq, mq, _, _, _ = sg.sg_prune_quantize_layer(W, Hinv, "0.5", 8, B, mask_in=mp)
    torch.cuda.synchronize()
    assert torch.equal(mp, mq)
    assert _rel(Wq.cpu().numpy(), Wp.cpu().numpy()) <= 2e-2
