"""Full-size checks in the benchmark's launch configuration (one Hessian call
over all resident tokens, one factor call, one prune call per pattern),
against the fp64 oracle at every width.

4096- and 11008-wide layers: the oracle H is computed in full on the host
from the same bf16 bytes, and the oracle U from it.  28672-wide layer: H on
a contiguous 2048-channel block and a channel sample from X's columns, and
the oracle U of the GPU's own H (the factor kernel's input) against the
GPU's U in full.

Unstructured masks couple all rows, so on sampled rows the check is that the
GPU mask is a valid selection under the oracle's saliencies along the GPU's
own trajectory (near-ties allowed) and that W_hat matches the oracle with that
mask forced.  N:M rows are independent: sampled rows are run through the
oracle free and compared directly (per-row agreement, then W_hat with the
GPU's mask forced).  Reconstruction error through the undamped H on the
sampled rows: GPU W_hat against the oracle's W_hat.
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
_state = {}


def _say(msg):
    sys.stderr.write(f"[gpu-case] {msg}\n")
    sys.stderr.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    _say(request.node.nodeid)
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


def _run_layer(sg, name):
    """GPU pipeline for one workload, cached per module."""
    if name in _state:
        return _state[name]
    cfg = synth.CONFIGS[name]
    xsrc = cfg.x_source or name
    if xsrc in _state and "X" in _state[xsrc]:
        X = _state[xsrc]["X"]
    else:
        X = synth.make_x(cfg, "cuda")
    W = synth.make_weight(cfg, "cuda")
    _say(f"{name}: m={cfg.m} n={cfg.n} T={X.shape[0]} H / factor / prune")
    H = torch.zeros(cfg.n, cfg.n, device="cuda")
    sg.sg_hessian_accumulate(H, X)
    Hinv, info = sg.sg_prepare_hinv(H, cfg.damp)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    res = {"cfg": cfg, "X": X, "W": W, "H": H, "Hinv": Hinv, "prune": {}}
    for p in cfg.patterns:
        Wh, mask = sg.sg_prune_layer(W, Hinv, p, cfg.blocksize)
        torch.cuda.synchronize()
        res["prune"][p] = (Wh, mask)
    _state[name] = res
    return res


def _oracle_H_full(X):
    """oracle H from the device X, one 32768-token chunk at a time (widened
    to fp64 exactly, then copied to the host)."""
    return oracle.hessian(X[t:t + 32768].double().cpu().numpy() for t in range(0, X.shape[0], 32768))


def _check_counts_and_zeros(W_hat, mask, pattern, B):
    m, n = mask.shape
    gm = mask.cpu().numpy().astype(bool)
    Wh = W_hat.cpu().numpy()
    assert np.all(Wh[gm] == 0.0) and not np.any(np.signbit(Wh[gm]))
    if ":" in pattern:
        N, M = map(int, pattern.split(":"))
        assert np.all(gm.reshape(m, -1, M).sum(axis=2) == M - N)
    else:
        p = float(pattern)
        for j in range(0, n, B):
            w = min(B, n - j)
            assert int(gm[:, j:j + w].sum()) == math.floor(p * m * w)
    return gm, Wh


def _consistency(S, gmask, pattern, B, across_rows):
    """Pruned saliencies never exceed kept ones (relative gap TAU)."""
    m, n = gmask.shape
    if ":" in pattern:
        M = int(pattern.split(":")[1])
        for j in range(0, n, M):
            s, g = S[:, j:j + M], gmask[:, j:j + M]
            hi = np.where(g, s, -np.inf).max(axis=1)
            lo = np.where(~g, s, np.inf).min(axis=1)
            assert not np.any(hi > lo * (1 + TAU) + 1e-300), f"group {j}"
    else:
        for j in range(0, n, B):
            s, g = S[:, j:j + B], gmask[:, j:j + B]
            if across_rows and g.any() and (~g).any():
                assert s[g].max() <= s[~g].min() * (1 + TAU) + 1e-300, f"block {j}"


# ---------------------------------------------------------------------------
# 4096-wide layers: full oracle H and U
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def attn_oracle(sg):
    res = _run_layer(sg, "attn_4096")
    if "oracle" not in res:
        _say("attn_4096: fp64 oracle H and U on the host")
        H = _oracle_H_full(res["X"])
        Hd, lam = oracle.dampen(H, res["cfg"].damp)
        res["oracle"] = {"H": H, "U": oracle.inverse_upper_factor(Hd), "lam": lam}
    return res


def test_attn_4096_hessian_and_factor(attn_oracle):
    res = attn_oracle
    Hg = res["H"].cpu().double().numpy()
    assert np.array_equal(Hg, Hg.T)
    assert _rel(Hg, res["oracle"]["H"]) <= 1e-5
    Ug = res["Hinv"].cpu().double().numpy()
    assert np.all(np.tril(Ug, -1) == 0.0)
    assert _rel(Ug, res["oracle"]["U"]) <= 1e-4


def test_attn_4096_unstructured_rows(attn_oracle):
    res = attn_oracle
    cfg = res["cfg"]
    p = cfg.patterns[0]
    Wh, mask = res["prune"][p]
    gm, Whg = _check_counts_and_zeros(Wh, mask, p, cfg.blocksize)
    rows = np.random.default_rng(7).choice(cfg.m, 48, replace=False)
    Wd = res["W"].cpu().double().numpy()[rows]
    U = res["oracle"]["U"]
    Who, _, _, tr = oracle.prune(Wd, U, p, cfg.blocksize, mask_in=gm[rows], return_trace=True)
    _consistency(tr["saliency"], gm[rows], p, cfg.blocksize, across_rows=True)
    assert _rel(Whg[rows], Who) <= 1e-4


def test_mlp_up_11008_nm_rows(sg, attn_oracle):
    res = _run_layer(sg, "mlp_up_11008")
    cfg = res["cfg"]
    p = cfg.patterns[0]
    Wh, mask = res["prune"][p]
    gm, Whg = _check_counts_and_zeros(Wh, mask, p, cfg.blocksize)
    U = attn_oracle["oracle"]["U"]  # same activations, same H and U
    rows = np.random.default_rng(8).choice(cfg.m, 64, replace=False)
    Wd = res["W"].cpu().double().numpy()[rows]
    Who, Mo, _ = oracle.prune(Wd, U, p, cfg.blocksize)
    agree = (gm[rows] == Mo).mean(axis=1)
    assert agree.min() >= 0.995
    Whf, _, _, tr = oracle.prune(Wd, U, p, cfg.blocksize, mask_in=gm[rows], return_trace=True)
    _consistency(tr["saliency"], gm[rows], p, cfg.blocksize, across_rows=False)
    assert _rel(Whg[rows], Whf) <= 1e-4
    # reconstruction error of the sampled rows against the oracle's own W_hat
    Hd_full = attn_oracle["oracle"]["H"]
    E_gpu = oracle.reconstruction_error_from_hessian(Wd, Whg[rows], Hd_full)
    E_o = oracle.reconstruction_error_from_hessian(Wd, Who, Hd_full)
    assert abs(E_gpu - E_o) <= 1e-3 * E_o
    # 2:4 compressed export of the whole layer; sampled rows against the oracle
    _say("mlp_up_11008: 2:4 export")
    vo, mo, bo = oracle.pack_two_four(Whg[rows], gm[rows])
    assert bo == 0
    for vdt in (torch.float32, torch.bfloat16):
        vals, meta, bad = sg.sg_pack_two_four(Wh, mask, value_dtype=vdt)
        torch.cuda.synchronize()
        assert int(bad.item()) == 0
        ri = torch.from_numpy(rows).cuda()
        vg = vals.index_select(0, ri).cpu()
        want = torch.from_numpy(vo.astype(np.float32)).to(vdt)
        iv = torch.int16 if vdt == torch.bfloat16 else torch.int32
        assert torch.equal(vg.view(iv), want.view(iv))
        assert np.array_equal(meta.index_select(0, ri).cpu().numpy(), mo)


def test_mlp_up_11008_quantized_rows(sg, attn_oracle):
    # joint 2:4 + 4-bit sweep at full size; rows are independent under N:M, so
    # sampled rows go through the oracle along the GPU's own trajectory
    res = _run_layer(sg, "mlp_up_11008")
    cfg = res["cfg"]
    Wh, mask, codes, scale, zero = sg.sg_prune_quantize_layer(res["W"], res["Hinv"], "2:4", 4,
                                                              cfg.blocksize)
    torch.cuda.synchronize()
    gm, Whg = _check_counts_and_zeros(Wh, mask, "2:4", cfg.blocksize)
    rows = np.random.default_rng(9).choice(cfg.m, 48, replace=False)
    Wd = res["W"].cpu().double().numpy()[rows]
    U = attn_oracle["oracle"]["U"]
    so, zo = oracle.quant_grid(Wd, 4)
    sc = scale.cpu().numpy()[rows]
    assert np.abs(sc - so).max() <= 1e-6 * np.abs(so).max()
    assert np.array_equal(zero.cpu().numpy()[rows].astype(np.float64), zo)
    cg = codes.cpu().numpy()[rows]
    Whf, _, _, _, _, _, tr = oracle.prune_quantized(Wd, U, "2:4", cfg.blocksize, 4, mask_in=gm[rows],
                                                    codes_in=cg, return_trace=True)
    _consistency(tr["saliency"], gm[rows], "2:4", cfg.blocksize, across_rows=False)
    y = tr["at_quant"] / so[:, None]
    near = np.abs(y - np.floor(y) - 0.5) <= 1e-4
    want = oracle.quant_code(tr["at_quant"], so[:, None], zo[:, None], 4)
    assert not np.any((~gm[rows]) & (cg != want) & ~near)
    assert _rel(Whg[rows], Whf) <= 1e-4


# ---------------------------------------------------------------------------
# wide layers
# ---------------------------------------------------------------------------

def _rows_checks(res, pattern, U, H_e, nrows, seed):
    """Sampled rows of one pattern against the oracle with factor U; the
    reconstruction error through H_e (undamped)."""
    cfg = res["cfg"]
    B = cfg.blocksize
    Wh, mask = res["prune"][pattern]
    gm, Whg = _check_counts_and_zeros(Wh, mask, pattern, B)
    rows = np.sort(np.random.default_rng(seed).choice(cfg.m, nrows, replace=False))
    Wd = res["W"].index_select(0, torch.from_numpy(rows).cuda()).double().cpu().numpy()
    Whr = Whg[rows].astype(np.float64)
    g = gm[rows]
    Whf, _, _, tr = oracle.prune(Wd, U, pattern, B, mask_in=g, return_trace=True)
    _consistency(tr["saliency"], g, pattern, B, across_rows=":" not in pattern)
    assert _rel(Whr, Whf) <= 1e-4
    if ":" in pattern:
        Who, Mo, _ = oracle.prune(Wd, U, pattern, B)
        agree = (g == Mo).mean(axis=1)
        _say(f"{cfg.name} {pattern}: per-row mask agreement min {agree.min():.5f} "
             f"mean {agree.mean():.5f}")
        assert agree.min() >= 0.995
    else:
        Who = Whf  # block-global selection: the oracle's W_hat on the GPU's mask
    E_gpu = oracle.reconstruction_error_from_hessian(Wd, Whr, H_e)
    E_o = oracle.reconstruction_error_from_hessian(Wd, Who, H_e)
    assert abs(E_gpu - E_o) <= 1e-3 * E_o


def _oracle_H_block(X, cols):
    """oracle H of the channels `cols` (a 1-D index tensor on the device)."""
    chunks = (X[t:t + 32768].index_select(1, cols).double().cpu().numpy()
              for t in range(0, X.shape[0], 32768))
    return oracle.hessian(chunks)


def test_mlp_down_11008_oracle(sg):
    """4096 x 11008 (60% unstructured and 4:8): full H and U against the
    oracle's; sampled rows of both patterns against the oracle with its U."""
    for k in list(_state):
        if k != "mlp_down_11008":
            _state.pop(k)
    torch.cuda.empty_cache()
    res = _run_layer(sg, "mlp_down_11008")
    cfg = res["cfg"]
    _say("mlp_down_11008: fp64 oracle H and U on the host")
    Ho = _oracle_H_full(res["X"])
    Hg = res["H"].cpu().double().numpy()
    assert np.array_equal(Hg, Hg.T)
    assert _rel(Hg, Ho) <= 1e-5
    del Hg
    Hd, _ = oracle.dampen(Ho, cfg.damp)
    Uo = oracle.inverse_upper_factor(Hd)
    del Hd
    Ug = res["Hinv"].cpu().double().numpy()
    assert np.all(np.tril(Ug, -1) == 0.0)
    err_u = _rel(Ug, Uo)
    _say(f"mlp_down_11008: U rel err {err_u:.3e}")
    assert err_u <= 1e-4
    del Ug
    for i, p in enumerate(cfg.patterns):
        _say(f"mlp_down_11008 pattern {p}: sampled rows against the oracle")
        _rows_checks(res, p, Uo, Ho, 64, 30 + i)
    _state.pop("mlp_down_11008", None)
    torch.cuda.empty_cache()


def test_mlp_down_28672_oracle(sg):
    """8192 x 28672 (50% unstructured and 2:4): H on a contiguous 2048-channel
    block and a channel sample against the definition from X's columns; the
    oracle U of the GPU's H against the GPU's U in full; sampled rows of both
    patterns against the oracle with that U."""
    for k in list(_state):
        _state.pop(k)
    torch.cuda.empty_cache()
    res = _run_layer(sg, "mlp_down_28672")
    cfg = res["cfg"]
    X, n = res["X"], cfg.n
    rng = np.random.default_rng(11)
    _say("mlp_down_28672: H on a 2048-channel block and 40 sampled channels")
    c0 = 13312
    for cols in (np.arange(c0, c0 + 2048), np.sort(rng.choice(n, 40, replace=False))):
        idx = torch.from_numpy(cols).cuda()
        Hs = _oracle_H_block(X, idx)
        Hg = res["H"].index_select(0, idx).index_select(1, idx).cpu().double().numpy()
        assert _rel(Hg, Hs) <= 1e-5
    del res["X"], X
    torch.cuda.empty_cache()
    _say("mlp_down_28672: fp64 oracle U of the GPU's H on the host")
    H_e = res["H"].cpu().double().numpy()
    Hd, _ = oracle.dampen(H_e, cfg.damp)
    Uo = oracle.inverse_upper_factor(Hd)
    del Hd
    Ug = res["Hinv"].cpu().double().numpy()
    assert np.all(np.tril(Ug, -1) == 0.0)
    err_u = _rel(Ug, Uo)
    _say(f"mlp_down_28672: U rel err {err_u:.3e}")
    assert err_u <= 1e-4
    del Ug
    for i, p in enumerate(cfg.patterns):
        _say(f"mlp_down_28672 pattern {p}: sampled rows against the oracle")
        _rows_checks(res, p, Uo, H_e, 32, 40 + i)
    _state.pop("mlp_down_28672", None)
    torch.cuda.empty_cache()
