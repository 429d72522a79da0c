"""Matrices that share one input, pruned in one call (sg_prune_layers_shared).

Each matrix's rows must equal its own single-matrix call bit for bit (the same
keys, counts and per-row arithmetic), and against the fp64 oracle each matrix
is its own layer: exact per-matrix counts, per-row mask agreement >= 99.5%,
selections consistent with the oracle's saliencies along the GPU trajectory
and W_hat within 1e-4 relative with the mask forced.
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
def layer(sg):
    n, T, B = 512, 8192, 128
    rows = (256, 130, 200)
    cfg = synth.LayerConfig("shared", sum(rows), n, T, 0.02, "bf16", "linear", 8, 20.0, ("0.5",), B,
                            config_id=970, chunk_tokens=T)
    W = synth.make_weight(cfg, "cpu")
    X = synth.make_x(cfg, "cpu")
    H = oracle.hessian([X.double().numpy()])
    Hd, _ = oracle.dampen(H, cfg.damp)
    U = oracle.inverse_upper_factor(Hd)
    Hg = torch.zeros(n, n, device="cuda")
    sg.sg_hessian_accumulate(Hg, X.cuda())
    Hinv, info = sg.sg_prepare_hinv(Hg, cfg.damp)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    splits = [0]
    for r in rows:
        splits.append(splits[-1] + r)
    return {"W": W, "Wc": W.cuda(), "U": U, "Hinv": Hinv, "splits": splits, "B": B}


@pytest.mark.parametrize("pattern,bits", [("0.5", 0), ("0.6", 0), ("2:4", 0), ("0.5/row", 0),
                                          ("0.5", 4), ("16:32", 3)])
def test_shared_equals_separate_calls(sg, layer, pattern, bits):
    Wc, Hinv, sp, B = layer["Wc"], layer["Hinv"], layer["splits"], layer["B"]
    out = sg.sg_prune_layers_shared(Wc, sp, Hinv, pattern, B, bits=bits)
    torch.cuda.synchronize()
    for p in range(len(sp) - 1):
        Wp = Wc[sp[p]:sp[p + 1]].contiguous()
        if bits:
            ref = sg.sg_prune_quantize_layer(Wp, Hinv, pattern, bits, B)
        else:
            ref = sg.sg_prune_layer(Wp, Hinv, pattern, B)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            if a.dim() == 2:
                assert torch.equal(a[sp[p]:sp[p + 1]], b), f"matrix {p}"
            else:
                assert torch.equal(a[sp[p]:sp[p + 1]], b), f"matrix {p} (row grid)"


def test_shared_unstructured_against_oracle(sg, layer):
    W, U, Hinv, sp, B = layer["W"], layer["U"], layer["Hinv"], layer["splits"], layer["B"]
    Wh, mask = sg.sg_prune_layers_shared(layer["Wc"], sp, Hinv, "0.5", B)
    torch.cuda.synchronize()
    Whg = Wh.cpu().numpy()
    gm = mask.cpu().numpy().astype(bool)
    Wd = W.double().numpy()
    n = Wd.shape[1]
    for p in range(len(sp) - 1):
        sl = slice(sp[p], sp[p + 1])
        mp = sp[p + 1] - sp[p]
        for j in range(0, n, B):
            w = min(B, n - j)
            assert int(gm[sl, j:j + w].sum()) == math.floor(0.5 * mp * w)
        Who, Mo, _ = oracle.prune(Wd[sl], U, "0.5", B)
        assert (gm[sl] == Mo).mean(axis=1).min() >= 0.995
        Whf, _, _, tr = oracle.prune(Wd[sl], U, "0.5", B, mask_in=gm[sl], return_trace=True)
        S = tr["saliency"]
        for j in range(0, n, B):
            s, g = S[:, j:j + B], gm[sl, j:j + B]
            if g.any() and (~g).any():
                assert s[g].max() <= s[~g].min() * (1 + TAU) + 1e-300
        assert _rel(Whg[sl], Whf) <= 1e-4
