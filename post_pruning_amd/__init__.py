"""SparseGPT layer solver for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libsg.so`` (declared in include/sg.h).
The functions carry the same names as the C entry points; they only marshal
torch tensors (device memory and the current HIP stream) into the calls.  All
arithmetic runs in the library's HIP kernels: there is no fallback, and every
call raises if the library is missing or the device is not gfx950.

Pipeline for one linear layer (W: m x n, calibration X token-major [N, n]):

    H = torch.zeros(n, n, device="cuda")
    for Xc in chunks: sg_hessian_accumulate(H, Xc)
    Hinv, info = sg_prepare_hinv(H, damp=0.01)
    W_hat, mask = sg_prune_layer(W, Hinv, 0.5 or "2:4", blocksize=128)
    err = sg_reconstruction_error(W, W_hat, Xc)      # optional validation
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsg.so")

SG_OK, SG_ERR_INVALID_ARGUMENT, SG_ERR_UNSUPPORTED, SG_ERR_WORKSPACE, SG_ERR_HIP = range(5)
SG_F32, SG_BF16 = 0, 1
SG_UNSTRUCTURED, SG_NM, SG_UNSTRUCTURED_ROW = 0, 1, 2
SG_OP_HESSIAN, SG_OP_PREPARE_HINV, SG_OP_PRUNE, SG_OP_RECON = range(4)
SG_MAX_BLOCKSIZE = 128
SG_MAX_SEGMENTS = 16
SG_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class SGError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsg.so (built by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    c_i32, c_i64, c_sz, c_vp, c_dbl = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                        ctypes.c_void_p, ctypes.c_double)
    lib.sg_hessian_accumulate.argtypes = [c_vp, c_i64, c_vp, c_i32, c_i64, c_i64, c_vp, c_sz, c_vp]
    lib.sg_prepare_hinv.argtypes = [c_vp, c_vp, c_i64, c_dbl, c_vp, c_vp, c_sz, c_vp, c_vp, c_vp, c_vp]
    lib.sg_prune_layer.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_i32,
                                   c_dbl, c_i32, c_i32, c_i32, c_vp, c_vp, c_sz, c_vp]
    lib.sg_reconstruction_error.argtypes = [c_vp, c_i32, c_vp, c_i32, c_i64, c_vp, c_i64, c_i64,
                                            c_vp, c_i32, c_i64, c_i64, c_vp, c_sz, c_vp]
    lib.sg_pack_two_four.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp]
    lib.sg_prune_quantize_layer.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                            c_i64, c_i64, c_vp, c_i32, c_dbl, c_i32, c_i32, c_i32,
                                            c_vp, c_vp, c_sz, c_vp]
    lib.sg_prune_layers_shared.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                           c_i64, c_i64, c_vp, c_i32, c_vp, c_i32, c_dbl, c_i32,
                                           c_i32, c_i32, c_vp, c_vp, c_sz, c_vp]
    lib.sg_prune_layer_noalloc.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_i32,
                                           c_dbl, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.sg_prune_layers_batched.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_i64,
                                            c_i64, c_i64, c_vp, c_i32, c_vp, c_i32, c_dbl, c_i32,
                                            c_i32, c_i32, c_vp, c_vp, c_sz, c_vp]
    lib.sg_prepare_hinv_batched.argtypes = [c_vp, c_vp, c_i32, c_i64, c_dbl, c_vp, c_vp, c_sz, c_vp, c_vp,
                                            c_vp, c_vp]
    lib.sg_prune_layer_vector.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_i32,
                                          c_dbl, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_sz, c_vp]
    for f in ("sg_hessian_accumulate", "sg_prepare_hinv", "sg_prune_layer",
              "sg_reconstruction_error", "sg_pack_two_four", "sg_prune_quantize_layer",
              "sg_prune_layers_shared", "sg_prune_layer_vector", "sg_prune_layer_noalloc",
              "sg_prune_layers_batched", "sg_prepare_hinv_batched"):
        getattr(lib, f).restype = c_i32
    lib.sg_workspace_bytes.argtypes = [c_i32, c_i64, c_i64, c_i64, c_i32]
    lib.sg_workspace_bytes.restype = c_sz
    lib.sg_status_string.argtypes = [c_i32]
    lib.sg_status_string.restype = ctypes.c_char_p
    lib.sg_last_error_message.argtypes = []
    lib.sg_last_error_message.restype = ctypes.c_char_p
    lib.sg_abi_version.argtypes = []
    lib.sg_abi_version.restype = c_i32
    _lib = lib
    return lib


def sg_abi_version() -> int:
    return int(load_library().sg_abi_version())


def sg_status_string(s: int) -> str:
    return load_library().sg_status_string(int(s)).decode()


def sg_last_error_message() -> str:
    return load_library().sg_last_error_message().decode()


def sg_workspace_bytes(op: int, m: int = 0, n: int = 0, T: int = 0, blocksize: int = 0) -> int:
    return int(load_library().sg_workspace_bytes(op, m, n, T, blocksize))


def _check(status: int, where: str):
    if status != SG_OK:
        raise SGError(status, where, sg_last_error_message() or sg_status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SG_F32
    if t.dtype == torch.bfloat16:
        return SG_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _row_major(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor (unit column stride)")
    return t.stride(0)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace of {nbytes} bytes needed")
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return ws, nbytes


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def sg_hessian_accumulate(H: torch.Tensor, X: torch.Tensor,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H += X^T X for a token-major chunk X [T, n] (bf16 or fp32); H is [n, n] fp32."""
    lib = load_library()
    _require_cuda(H, X)
    if H.dtype != torch.float32 or not H.is_contiguous() or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise ValueError("H must be a contiguous square float32 tensor")
    n = H.shape[0]
    if X.dim() != 2 or X.shape[1] != n:
        raise ValueError("X must be [T, n]")
    ldx = _row_major(X, "X")
    T = X.shape[0]
    need = sg_workspace_bytes(SG_OP_HESSIAN, 0, n, T, 0)
    ws, nb = _workspace(need, H.device, workspace)
    _check(lib.sg_hessian_accumulate(_ptr(H), n, _ptr(X), _dtype_code(X), T, ldx, _ptr(ws), nb,
                                     ctypes.c_void_p(_stream(H.device))), "sg_hessian_accumulate")
    return H


# Above this n the factorisation's trailing updates can run on a second stream
# (the library's fused single-stream form is used up to it either way).
FACTOR_SPLIT_MIN_N = 4097


def sg_prepare_hinv(H: torch.Tensor, damp: float = 0.01, Hinv: Optional[torch.Tensor] = None,
                    info: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    update_stream: Union[str, None, "torch.cuda.Stream"] = "auto",
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Upper Cholesky factor of (H + damp*mean(diag H) I)^{-1}; returns (Hinv, info).

    ``update_stream``: "auto" takes a stream from torch's pool and two fresh
    events for this call when n > 4096 (the trailing updates then overlap the
    panel chain); a torch.cuda.Stream uses that stream; None keeps every
    kernel on the current stream.  The library itself creates no stream."""
    lib = load_library()
    _require_cuda(H)
    n = H.shape[0]
    if H.dtype != torch.float32 or not H.is_contiguous() or H.shape != (n, n):
        raise ValueError("H must be a contiguous square float32 tensor")
    if Hinv is None:
        Hinv = torch.empty_like(H)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=H.device)
    need = sg_workspace_bytes(SG_OP_PREPARE_HINV, 0, n, 0, 0)
    ws, nb = _workspace(need, H.device, workspace)
    side = ev_a = ev_b = None
    if isinstance(update_stream, str):
        if update_stream != "auto":
            raise ValueError("update_stream must be 'auto', None or a torch.cuda.Stream")
        if n >= FACTOR_SPLIT_MIN_N:
            side = torch.cuda.Stream(device=H.device)
    else:
        side = update_stream
    if side is not None:
        # events owned by this call (created by their first record)
        ev_a, ev_b = torch.cuda.Event(), torch.cuda.Event()
        ev_a.record(side)
        ev_b.record(side)
    _check(lib.sg_prepare_hinv(_ptr(Hinv), _ptr(H), n, float(damp), _ptr(info), _ptr(ws), nb,
                               ctypes.c_void_p(_stream(H.device)),
                               None if side is None else ctypes.c_void_p(side.cuda_stream),
                               None if ev_a is None else ctypes.c_void_p(ev_a.cuda_event),
                               None if ev_b is None else ctypes.c_void_p(ev_b.cuda_event)),
           "sg_prepare_hinv")
    return Hinv, info


def sg_prepare_hinv_batched(Hs, damp: float = 0.01, Hinvs=None, info: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None,
                            update_stream: Union[str, None, "torch.cuda.Stream"] = "auto"):
    """sg_prepare_hinv for several [n, n] matrices of one order n in one call;
    returns (Hinvs, info) with info an int32 tensor of one status per matrix.
    Each factor equals sg_prepare_hinv's of the same matrix, bit for bit."""
    lib = load_library()
    Hs = list(Hs)
    if not Hs:
        raise ValueError("at least one matrix")
    _require_cuda(*Hs)
    n = Hs[0].shape[0]
    for H in Hs:
        if H.dtype != torch.float32 or not H.is_contiguous() or H.shape != (n, n):
            raise ValueError("every H must be a contiguous square float32 tensor of the same order")
    nl = len(Hs)
    dev = Hs[0].device
    if Hinvs is None:
        Hinvs = [torch.empty_like(H) for H in Hs]
    if info is None:
        info = torch.empty(nl, dtype=torch.int32, device=dev)
    need = nl * sg_workspace_bytes(SG_OP_PREPARE_HINV, 0, n, 0, 0)
    ws, nb = _workspace(need, dev, workspace)
    side = ev_a = ev_b = None
    if isinstance(update_stream, str):
        if update_stream != "auto":
            raise ValueError("update_stream must be 'auto', None or a torch.cuda.Stream")
        if n >= FACTOR_SPLIT_MIN_N:
            side = torch.cuda.Stream(device=dev)
    else:
        side = update_stream
    if side is not None:
        ev_a, ev_b = torch.cuda.Event(), torch.cuda.Event()
        ev_a.record(side)
        ev_b.record(side)
    hp = (ctypes.c_void_p * nl)(*[h.data_ptr() for h in Hs])
    up = (ctypes.c_void_p * nl)(*[u.data_ptr() for u in Hinvs])
    _check(lib.sg_prepare_hinv_batched(ctypes.cast(up, ctypes.c_void_p), ctypes.cast(hp, ctypes.c_void_p), nl, n,
                                       float(damp), _ptr(info), _ptr(ws), nb, ctypes.c_void_p(_stream(dev)),
                                       None if side is None else ctypes.c_void_p(side.cuda_stream),
                                       None if ev_a is None else ctypes.c_void_p(ev_a.cuda_event),
                                       None if ev_b is None else ctypes.c_void_p(ev_b.cuda_event)),
           "sg_prepare_hinv_batched")
    return Hinvs, info


def parse_pattern(pattern: Union[float, str]):
    """0.5 -> (SG_UNSTRUCTURED, 0.5, 0, 1); "0.5/row" -> (SG_UNSTRUCTURED_ROW,
    0.5, 0, 1); "2:4" -> (SG_NM, 0.0, 2, 4)."""
    if isinstance(pattern, str) and ":" in pattern:
        a, b = pattern.split(":")
        return SG_NM, 0.0, int(a), int(b)
    if isinstance(pattern, str) and pattern.endswith("/row"):
        return SG_UNSTRUCTURED_ROW, float(pattern[:-4]), 0, 1
    return SG_UNSTRUCTURED, float(pattern), 0, 1


def sg_prune_layer(W: torch.Tensor, Hinv: torch.Tensor, pattern: Union[float, str],
                   blocksize: int = 128, mask_in: Optional[torch.Tensor] = None,
                   W_out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """Prune W ([m, n] bf16/fp32) with the factor Hinv; returns (W_hat fp32, mask uint8)."""
    lib = load_library()
    _require_cuda(W, Hinv, mask_in)
    m, n = W.shape
    ldw = _row_major(W, "W")
    if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous():
            raise ValueError("mask_in must be a contiguous [m, n] tensor")
        mask_in = mask_in.to(torch.uint8)
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    need = sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize)
    ws, nb = _workspace(need, W.device, workspace)
    _check(lib.sg_prune_layer(_ptr(W_out), _ptr(mask_out), _ptr(W), _dtype_code(W), m, n, ldw,
                              _ptr(Hinv), kind, sp, nk, mg, int(blocksize), _ptr(mask_in), _ptr(ws),
                              nb, ctypes.c_void_p(_stream(W.device))), "sg_prune_layer")
    return W_out, mask_out


def sg_prune_layer_noalloc(W: torch.Tensor, Hinv: torch.Tensor, pattern: Union[float, str],
                           blocksize: int = 128, mask_in: Optional[torch.Tensor] = None,
                           W_out: Optional[torch.Tensor] = None,
                           mask_out: Optional[torch.Tensor] = None):
    """sg_prune_layer with the library's per-GPU scratch array in place of a
    workspace (the C call allocates nothing; pass W_out and mask_out to keep
    this wrapper from allocating them).  Calls overlapping on one GPU race."""
    lib = load_library()
    _require_cuda(W, Hinv, mask_in)
    m, n = W.shape
    ldw = _row_major(W, "W")
    if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous() or mask_in.dtype != torch.uint8:
            raise ValueError("mask_in must be a contiguous [m, n] uint8 tensor")
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    _check(lib.sg_prune_layer_noalloc(_ptr(W_out), _ptr(mask_out), _ptr(W), _dtype_code(W), m, n, ldw,
                                      _ptr(Hinv), kind, sp, nk, mg, int(blocksize), _ptr(mask_in),
                                      ctypes.c_void_p(_stream(W.device))), "sg_prune_layer_noalloc")
    return W_out, mask_out


def sg_prune_layer_vector(W: torch.Tensor, Hinv: torch.Tensor, pattern: Union[float, str], vec: int = 16,
                          blocksize: int = 128, mask_in: Optional[torch.Tensor] = None,
                          W_out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """Prune W with the chosen weights of each range of ``vec`` columns removed
    together (vec = 16; vec = 1 is sg_prune_layer); returns (W_hat, mask)."""
    lib = load_library()
    _require_cuda(W, Hinv, mask_in)
    m, n = W.shape
    ldw = _row_major(W, "W")
    if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous():
            raise ValueError("mask_in must be a contiguous [m, n] tensor")
        mask_in = mask_in.to(torch.uint8)
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    need = sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize)
    ws, nb = _workspace(need, W.device, workspace)
    _check(lib.sg_prune_layer_vector(_ptr(W_out), _ptr(mask_out), _ptr(W), _dtype_code(W), m, n, ldw,
                                     _ptr(Hinv), kind, sp, nk, mg, int(blocksize), int(vec),
                                     _ptr(mask_in), _ptr(ws), nb, ctypes.c_void_p(_stream(W.device))),
           "sg_prune_layer_vector")
    return W_out, mask_out


def sg_prune_quantize_layer(W: torch.Tensor, Hinv: torch.Tensor, pattern: Union[float, str], bits: int,
                            blocksize: int = 128, mask_in: Optional[torch.Tensor] = None,
                            W_out: Optional[torch.Tensor] = None,
                            mask_out: Optional[torch.Tensor] = None,
                            codes_out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None):
    """Prune W and round its kept weights to a per-row grid of 2^bits levels in
    one sweep; returns (W_hat fp32, mask uint8, codes uint8, scale fp32 [m],
    zero fp32 [m]) with W_hat = scale * (codes - zero)."""
    lib = load_library()
    _require_cuda(W, Hinv, mask_in)
    m, n = W.shape
    ldw = _row_major(W, "W")
    if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous():
            raise ValueError("mask_in must be a contiguous [m, n] tensor")
        mask_in = mask_in.to(torch.uint8)
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    if codes_out is None:
        codes_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    scale = torch.empty(m, dtype=torch.float32, device=W.device)
    zero = torch.empty(m, dtype=torch.float32, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    need = sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize)
    ws, nb = _workspace(need, W.device, workspace)
    _check(lib.sg_prune_quantize_layer(_ptr(W_out), _ptr(mask_out), _ptr(codes_out), _ptr(scale),
                                       _ptr(zero), int(bits), _ptr(W), _dtype_code(W), m, n, ldw,
                                       _ptr(Hinv), kind, sp, nk, mg, int(blocksize), _ptr(mask_in),
                                       _ptr(ws), nb, ctypes.c_void_p(_stream(W.device))),
           "sg_prune_quantize_layer")
    return W_out, mask_out, codes_out, scale, zero


def sg_prune_layers_shared(W: torch.Tensor, row_splits, Hinv: torch.Tensor,
                           pattern: Union[float, str], blocksize: int = 128, bits: int = 0,
                           mask_in: Optional[torch.Tensor] = None,
                           W_out: Optional[torch.Tensor] = None,
                           mask_out: Optional[torch.Tensor] = None,
                           codes_out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None):
    """Prune matrices that share one input (stacked by rows in W, matrix p =
    rows row_splits[p]:row_splits[p+1]) with their shared factor in one call.

    Returns (W_hat, mask), or (W_hat, mask, codes, scale, zero) for bits > 0;
    each matrix's rows equal its own sg_prune_layer / sg_prune_quantize_layer
    result."""
    lib = load_library()
    _require_cuda(W, Hinv, mask_in)
    m, n = W.shape
    ldw = _row_major(W, "W")
    splits = [int(x) for x in row_splits]
    nseg = len(splits) - 1
    if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
        raise ValueError("Hinv must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous():
            raise ValueError("mask_in must be a contiguous [m, n] tensor")
        mask_in = mask_in.to(torch.uint8)
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    scale = zero = None
    if bits:
        if codes_out is None:
            codes_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
        scale = torch.empty(m, dtype=torch.float32, device=W.device)
        zero = torch.empty(m, dtype=torch.float32, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    need = sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize)
    ws, nb = _workspace(need, W.device, workspace)
    arr = (ctypes.c_int64 * max(1, len(splits)))(*splits)
    _check(lib.sg_prune_layers_shared(_ptr(W_out), _ptr(mask_out), _ptr(codes_out), _ptr(scale),
                                      _ptr(zero), int(bits), _ptr(W), _dtype_code(W), m, n, ldw,
                                      ctypes.cast(arr, ctypes.c_void_p), nseg, _ptr(Hinv), kind, sp,
                                      nk, mg, int(blocksize), _ptr(mask_in), _ptr(ws), nb,
                                      ctypes.c_void_p(_stream(W.device))), "sg_prune_layers_shared")
    if bits:
        return W_out, mask_out, codes_out, scale, zero
    return W_out, mask_out


def sg_prune_layers_batched(W: torch.Tensor, row_splits, Hinvs, pattern: Union[float, str],
                            blocksize: int = 128, bits: int = 0,
                            mask_in: Optional[torch.Tensor] = None,
                            W_out: Optional[torch.Tensor] = None,
                            mask_out: Optional[torch.Tensor] = None,
                            codes_out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None):
    """Prune several layers' matrices (stacked by rows in W, matrix p = rows
    row_splits[p]:row_splits[p+1]), matrix p with its own factor Hinvs[p], in
    one call.  Returns (W_hat, mask), or (W_hat, mask, codes, scale, zero) for
    bits > 0; each matrix's rows equal its own sg_prune_layer /
    sg_prune_quantize_layer result with its own factor."""
    lib = load_library()
    _require_cuda(W, mask_in, *Hinvs)
    m, n = W.shape
    ldw = _row_major(W, "W")
    splits = [int(x) for x in row_splits]
    nseg = len(splits) - 1
    if len(Hinvs) != nseg:
        raise ValueError("one factor per matrix")
    for Hinv in Hinvs:
        if Hinv.shape != (n, n) or Hinv.dtype != torch.float32 or not Hinv.is_contiguous():
            raise ValueError("every factor must be a contiguous [n, n] float32 tensor")
    if mask_in is not None:
        if mask_in.shape != (m, n) or not mask_in.is_contiguous():
            raise ValueError("mask_in must be a contiguous [m, n] tensor")
        mask_in = mask_in.to(torch.uint8)
    if W_out is None:
        W_out = torch.empty(m, n, dtype=torch.float32, device=W.device)
    if mask_out is None:
        mask_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
    scale = zero = None
    if bits:
        if codes_out is None:
            codes_out = torch.empty(m, n, dtype=torch.uint8, device=W.device)
        scale = torch.empty(m, dtype=torch.float32, device=W.device)
        zero = torch.empty(m, dtype=torch.float32, device=W.device)
    kind, sp, nk, mg = parse_pattern(pattern)
    need = sg_workspace_bytes(SG_OP_PRUNE, m, n, 0, blocksize)
    ws, nb = _workspace(need, W.device, workspace)
    arr = (ctypes.c_int64 * max(1, len(splits)))(*splits)
    ptrs = (ctypes.c_void_p * max(1, nseg))(*[h.data_ptr() for h in Hinvs])
    _check(lib.sg_prune_layers_batched(_ptr(W_out), _ptr(mask_out), _ptr(codes_out), _ptr(scale),
                                       _ptr(zero), int(bits), _ptr(W), _dtype_code(W), m, n, ldw,
                                       ctypes.cast(arr, ctypes.c_void_p), nseg,
                                       ctypes.cast(ptrs, ctypes.c_void_p), kind, sp, nk, mg,
                                       int(blocksize), _ptr(mask_in), _ptr(ws), nb,
                                       ctypes.c_void_p(_stream(W.device))), "sg_prune_layers_batched")
    if bits:
        return W_out, mask_out, codes_out, scale, zero
    return W_out, mask_out


def sg_reconstruction_error(W: torch.Tensor, W_hat: torch.Tensor, X: torch.Tensor,
                            err: Optional[torch.Tensor] = None, accumulate: bool = False,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """||(W - W_hat) X^T||_F^2 over a token-major chunk X; returns a device float64 scalar."""
    lib = load_library()
    _require_cuda(W, W_hat, X)
    m, n = W.shape
    ldw = _row_major(W, "W")
    ldx = _row_major(X, "X")
    if W_hat.shape != (m, n) or W_hat.dtype != torch.float32 or not W_hat.is_contiguous():
        raise ValueError("W_hat must be a contiguous [m, n] float32 tensor")
    if X.shape[1] != n:
        raise ValueError("X must be [T, n]")
    if err is None:
        err = torch.zeros(1, dtype=torch.float64, device=W.device)
    T = X.shape[0]
    need = sg_workspace_bytes(SG_OP_RECON, m, n, T, 0)
    ws, nb = _workspace(need, W.device, workspace)
    _check(lib.sg_reconstruction_error(_ptr(err), int(bool(accumulate)), _ptr(W), _dtype_code(W),
                                       ldw, _ptr(W_hat), m, n, _ptr(X), _dtype_code(X), T, ldx,
                                       _ptr(ws), nb, ctypes.c_void_p(_stream(W.device))),
           "sg_reconstruction_error")
    return err


def sg_pack_two_four(W_hat: torch.Tensor, mask: torch.Tensor,
                     value_dtype: torch.dtype = torch.float32,
                     values: Optional[torch.Tensor] = None, meta: Optional[torch.Tensor] = None):
    """2:4 compressed form of a pruned [m, n] matrix.

    Returns (values [m, n/2] of ``value_dtype`` (float32 or bfloat16),
    meta [m, ceil(n/8)] uint8, bad: device int32 count of groups with more than
    two kept positions)."""
    lib = load_library()
    _require_cuda(W_hat, mask)
    m, n = W_hat.shape
    if W_hat.dtype != torch.float32 or not W_hat.is_contiguous():
        raise ValueError("W_hat must be a contiguous float32 tensor")
    if mask.shape != (m, n) or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous [m, n] tensor")
    mask = mask.to(torch.uint8)
    if value_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("value_dtype must be float32 or bfloat16")
    if values is None:
        values = torch.empty(m, n // 2, dtype=value_dtype, device=W_hat.device)
    elif (values.shape != (m, n // 2) or values.dtype != value_dtype or not values.is_contiguous()
          or not values.is_cuda):
        raise ValueError("values must be a contiguous [m, n/2] GPU tensor of value_dtype")
    if meta is None:
        meta = torch.empty(m, (n + 7) // 8, dtype=torch.uint8, device=W_hat.device)
    elif meta.shape != (m, (n + 7) // 8) or meta.dtype != torch.uint8 or not meta.is_contiguous() \
            or not meta.is_cuda:
        raise ValueError("meta must be a contiguous [m, ceil(n/8)] uint8 GPU tensor")
    bad = torch.empty(1, dtype=torch.int32, device=W_hat.device)
    _check(lib.sg_pack_two_four(_ptr(values), _dtype_code(values), _ptr(meta), _ptr(bad),
                                _ptr(W_hat), _ptr(mask), m, n,
                                ctypes.c_void_p(_stream(W_hat.device))), "sg_pack_two_four")
    return values, meta, bad


def solve_layer(W: torch.Tensor, x_chunks, pattern, blocksize: int = 128, damp: float = 0.01):
    """a1..a7 for one layer: Hessian over all chunks, factor, prune."""
    n = W.shape[1]
    H = torch.zeros(n, n, dtype=torch.float32, device=W.device)
    for Xc in x_chunks:
        sg_hessian_accumulate(H, Xc)
    Hinv, info = sg_prepare_hinv(H, damp)
    W_hat, mask = sg_prune_layer(W, Hinv, pattern, blocksize)
    return {"H": H, "Hinv": Hinv, "info": info, "W_hat": W_hat, "mask": mask}
