"""Several layers, each with the factor of its own inputs, pruned in one call
(sg_prune_layers_batched).

Each matrix's rows must equal its own single-matrix call with its own factor
bit for bit (the same keys, counts and per-row arithmetic on its own U), and
against the fp64 oracle each matrix is its own layer with its own H and U:
exact per-matrix counts, per-row mask agreement >= 99.5%, selections
consistent with the oracle's saliencies along the GPU trajectory, W_hat
within 1e-4 relative with the mask forced, and the reconstruction error of
each layer within 1e-3 of the oracle's.
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


@pytest.fixture(scope="module")
def layers(sg):
    """Four layers of width 512 with their own activations (two linear, two
    post-activation) and weights of different heights."""
    n, T, B = 512, 8192, 128
    rows = (256, 130, 200, 64)
    acts = ("linear", "relu", "linear", "relu")
    Ws, Us, Hs, Hinvs = [], [], [], []
    for i, (r, act) in enumerate(zip(rows, acts)):
        cfg = synth.LayerConfig(f"batched_{i}", r, n, T, 0.02, "bf16", act, 8, 20.0, ("0.5",), B,
                                config_id=980 + i, chunk_tokens=T)
        W = synth.make_weight(cfg, "cpu")
        X = synth.make_x(cfg, "cpu")
        H = oracle.hessian([X.double().numpy()])
        Hd, _ = oracle.dampen(H, cfg.damp)
        Hg = torch.zeros(n, n, device="cuda")
        sg.sg_hessian_accumulate(Hg, X.cuda())
        Hinv, info = sg.sg_prepare_hinv(Hg, cfg.damp)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        Ws.append(W)
        Hs.append(H)
        Us.append(oracle.inverse_upper_factor(Hd))
        Hinvs.append(Hinv)
    splits = [0]
    for r in rows:
        splits.append(splits[-1] + r)
    Wall = torch.cat(Ws)
    return {"W": Wall, "Wc": Wall.cuda(), "U": Us, "H": Hs, "Hinv": Hinvs, "splits": splits, "B": B}


@pytest.mark.parametrize("pattern,bits", [("0.5", 0), ("0.6", 0), ("2:4", 0), ("0.5/row", 0),
                                          ("16:128", 0), ("0.5", 4), ("2:4", 3)])
def test_batched_equals_separate_calls(sg, layers, pattern, bits):
    Wc, Hinvs, sp, B = layers["Wc"], layers["Hinv"], layers["splits"], layers["B"]
    out = sg.sg_prune_layers_batched(Wc, sp, Hinvs, pattern, B, bits=bits)
    torch.cuda.synchronize()
    for p in range(len(sp) - 1):
        Wp = Wc[sp[p]:sp[p + 1]].contiguous()
        if bits:
            ref = sg.sg_prune_quantize_layer(Wp, Hinvs[p], pattern, bits, B)
        else:
            ref = sg.sg_prune_layer(Wp, Hinvs[p], pattern, B)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a[sp[p]:sp[p + 1]], b), f"matrix {p}"


@pytest.mark.parametrize("pattern", ["0.5", "2:4"])
def test_batched_against_oracle(sg, layers, pattern):
    W, sp, B = layers["W"], layers["splits"], layers["B"]
    Wh, mask = sg.sg_prune_layers_batched(layers["Wc"], sp, layers["Hinv"], pattern, B)
    torch.cuda.synchronize()
    Whg = Wh.cpu().numpy()
    gm = mask.cpu().numpy().astype(bool)
    Wd = W.double().numpy()
    n = Wd.shape[1]
    for p in range(len(sp) - 1):
        sl = slice(sp[p], sp[p + 1])
        mp = sp[p + 1] - sp[p]
        U = layers["U"][p]
        if ":" in pattern:
            assert np.all(gm[sl].reshape(mp, -1, 4).sum(axis=2) == 2)
        else:
            for j in range(0, n, B):
                w = min(B, n - j)
                assert int(gm[sl, j:j + w].sum()) == math.floor(0.5 * mp * w)
        Who, Mo, _ = oracle.prune(Wd[sl], U, pattern, B)
        assert (gm[sl] == Mo).mean(axis=1).min() >= 0.995
        Whf, _, _, tr = oracle.prune(Wd[sl], U, pattern, B, mask_in=gm[sl], return_trace=True)
        S = tr["saliency"]
        G = 4 if ":" in pattern else B
        for j in range(0, n, G):
            s, g = S[:, j:j + G], gm[sl, j:j + G]
            if ":" in pattern:
                hi = np.where(g, s, -np.inf).max(axis=1)
                lo = np.where(~g, s, np.inf).min(axis=1)
                assert not np.any(hi > lo * (1 + TAU) + 1e-300)
            elif g.any() and (~g).any():
                assert s[g].max() <= s[~g].min() * (1 + TAU) + 1e-300
        assert _rel(Whg[sl], Whf) <= 1e-4
        E_g = oracle.reconstruction_error_from_hessian(Wd[sl], Whg[sl], layers["H"][p])
        E_o = oracle.reconstruction_error_from_hessian(Wd[sl], Who, layers["H"][p])
        assert abs(E_g - E_o) <= 1e-3 * E_o
