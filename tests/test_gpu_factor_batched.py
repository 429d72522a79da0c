"""Several Hessians of one order factored in one call (sg_prepare_hinv_batched).

Each factor must equal the single-matrix sg_prepare_hinv of the same H bit for
bit (the same kernels on each layer's own part of the workspace), on every
route: the shared panel + update launch (n <= 4096), the grouped single-stream
route and the route with a caller update stream (n > 4096).  Against the fp64
oracle each factor is within 1e-4 relative of the textbook U of its own H, and
a layer whose factorisation fails (H = 0) reports its own info without
touching the others'.
"""

import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


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


def _hessians(sg, n, T, count, seed):
    """count Hessians of order n from bf16 activations with log-normal
    channel scales (different seeds per layer)."""
    Hs = []
    for i in range(count):
        g = torch.Generator(device="cpu").manual_seed(seed + i)
        X = (torch.randn(T, n, generator=g) * torch.exp(torch.randn(n, generator=g))).to(torch.bfloat16)
        H = torch.zeros(n, n, device="cuda")
        sg.sg_hessian_accumulate(H, X.cuda())
        Hs.append(H)
    torch.cuda.synchronize()
    return Hs


def _bits_equal(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("n,T,count,route", [
    (200, 2048, 3, "auto"),       # one block column, ragged
    (640, 4096, 4, "auto"),       # shared panel + update launches
    (4096, 16384, 2, "auto"),     # the attention layers' order
    (4224, 8192, 2, "auto"),      # caller update stream
    (4224, 8192, 3, None),        # grouped panels on one stream
    (256, 1024, 16, "auto"),      # the most layers one call takes
])
def test_batched_factor_equals_single_calls(sg, n, T, count, route):
    Hs = _hessians(sg, n, T, count, 7000 + n)
    Us, info = sg.sg_prepare_hinv_batched(Hs, 0.01, update_stream=route)
    torch.cuda.synchronize()
    assert info.tolist() == [0] * count
    for L, H in enumerate(Hs):
        U1, i1 = sg.sg_prepare_hinv(H, 0.01, update_stream=route)
        torch.cuda.synchronize()
        assert int(i1.item()) == 0
        assert _bits_equal(Us[L], U1), (n, L)


@pytest.mark.parametrize("n,count", [(640, 3), (1000, 2)])
def test_batched_factor_against_oracle(sg, n, count):
    Hs = _hessians(sg, n, 4096, count, 8100 + n)
    Us, info = sg.sg_prepare_hinv_batched(Hs, 0.01)
    torch.cuda.synchronize()
    assert info.tolist() == [0] * count
    for H, U in zip(Hs, Us):
        Hd, _ = oracle.dampen(H.double().cpu().numpy(), 0.01)
        Uo = oracle.inverse_upper_factor(Hd)
        Ug = U.double().cpu().numpy()
        assert np.all(np.tril(Ug, -1) == 0.0)
        assert np.linalg.norm(Ug - Uo) / np.linalg.norm(Uo) <= 1e-4


def test_batched_factor_info_per_layer(sg):
    """A zero Hessian in the middle reports n + 1 for itself only."""
    n = 384
    Hs = _hessians(sg, n, 2048, 3, 8300)
    Hs[1].zero_()
    Us, info = sg.sg_prepare_hinv_batched(Hs, 0.01)
    torch.cuda.synchronize()
    assert info.tolist() == [0, n + 1, 0]
    for L in (0, 2):
        U1, i1 = sg.sg_prepare_hinv(Hs[L], 0.01)
        torch.cuda.synchronize()
        assert _bits_equal(Us[L], U1)
