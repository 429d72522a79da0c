"""The no-allocation prune entry point against sg_prune_layer.

sg_prune_layer_noalloc runs the same kernels as sg_prune_layer with the
library's per-GPU scratch array in place of the caller's workspace, so its
results must equal sg_prune_layer's bit for bit.  Two calls in a row, the
second on a smaller input: whatever the first call left in the shared array
must not reach the second.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    import post_pruning_amd as sg
    sg.load_library()
    assert torch.cuda.is_available()
    return sg


def _layer(sg, name, m, n, tokens, pattern, B, seed):
    cfg = synth.LayerConfig(name, m, n, tokens, 0.02, "bf16", "linear", 4, 20.0, (pattern,), B,
                            config_id=seed, chunk_tokens=tokens)
    W = synth.make_weight(cfg, "cuda")
    X = synth.make_x(cfg, "cuda")
    H = torch.zeros(n, n, device="cuda")
    sg.sg_hessian_accumulate(H, X)
    Hinv, info = sg.sg_prepare_hinv(H, cfg.damp)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    return W, Hinv


def _noalloc_c(sg, W, Hinv, pattern, B, W_out, mask_out):
    """The C entry point called directly through ctypes."""
    lib = sg.load_library()
    m, n = W.shape
    kind, sp, nk, mg = sg.parse_pattern(pattern)
    st = lib.sg_prune_layer_noalloc(ctypes.c_void_p(W_out.data_ptr()), ctypes.c_void_p(mask_out.data_ptr()),
                                    ctypes.c_void_p(W.data_ptr()), sg.SG_BF16, m, n, W.stride(0),
                                    ctypes.c_void_p(Hinv.data_ptr()), kind, sp, nk, mg, B, None,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sg.sg_last_error_message()


def test_noalloc_matches_workspace_call_twice(sg):
    cases = [
        # (name, m, n, tokens, pattern, blocksize): the second is smaller
        ("noalloc_a", 384, 640, 8192, "0.5", 128),
        ("noalloc_b", 130, 384, 4096, "0.55", 64),
        ("noalloc_c", 96, 256, 4096, "2:4", 128),
    ]
    layers = [_layer(sg, c[0], c[1], c[2], c[3], c[4], c[5], 950 + i) for i, c in enumerate(cases)]
    for (name, m, n, _, pattern, B), (W, Hinv) in zip(cases, layers):
        sys.stderr.write(f"[gpu-case] no-alloc {name}: m={m} n={n} pattern={pattern} B={B}\n")
        sys.stderr.flush()
        ref_W, ref_mask = sg.sg_prune_layer(W, Hinv, pattern, B)
        W_out = torch.full((m, n), float("nan"), device="cuda")
        mask_out = torch.full((m, n), 7, dtype=torch.uint8, device="cuda")
        _noalloc_c(sg, W, Hinv, pattern, B, W_out, mask_out)
        torch.cuda.synchronize()
        assert torch.equal(W_out, ref_W), name
        assert torch.equal(mask_out, ref_mask), name
        gm = mask_out.cpu().numpy().astype(bool)
        if ":" not in pattern:
            for j in range(0, n, B):
                w = min(B, n - j)
                assert int(gm[:, j:j + w].sum()) == oracle.unstructured_k(float(pattern), m, w)
        # the binding's wrapper of the same call
        W2, M2 = sg.sg_prune_layer_noalloc(W, Hinv, pattern, B)
        torch.cuda.synchronize()
        assert torch.equal(W2, ref_W) and torch.equal(M2, ref_mask)


def test_noalloc_rejects_oversized(sg):
    W = torch.zeros(30000, 256, dtype=torch.bfloat16, device="cuda")
    Hinv = torch.eye(256, device="cuda")
    with pytest.raises(sg.SGError) as ei:
        sg.sg_prune_layer_noalloc(W, Hinv, 0.5, 128)
    assert ei.value.status == sg.SG_ERR_UNSUPPORTED
