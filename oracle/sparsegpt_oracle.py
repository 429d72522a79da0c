"""fp64 CPU oracle of the SparseGPT layer solver (test infrastructure only).

Every function below is the plain definition, or the algorithm's steps in the
pages' order, in float64 with numpy / PyTorch-CPU library primitives as steps.  No
blocking, batching or reordering beyond what the method itself states.

Notation: W is m x n (rows = output channels, columns = input channels, Y = WX);
calibration inputs are given token-major, X[t, c] (the transpose of the pages'
n x N matrix, i.e. the same bytes as a framework's activation tensor).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, Optional

import numpy as np
import torch


# ----------------------------------------------------------------------------
# Sparsity patterns
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Pattern:
    """A sparsity target.

    kind == "unstructured": prune a fraction ``sparsity`` of the weights
    ([SGR] section 11 step 5: the given fraction is pruned within each column
    block).  ``per_row`` False: the count is taken over the whole m x w block;
    ``per_row`` True: every row of the block prunes the same count on its own
    (the pages do not say which; both readings are offered).
    kind == "nm": keep ``n_keep`` of every ``m_group`` consecutive input
    columns of each row ([SFT] section 8.4: 2:4 keeps 2 of every 4, 16:64 keeps
    16 of every 64; [G24] 2:4 section: the zeros lie along the reduction axis).
    """

    kind: str
    sparsity: float = 0.0
    n_keep: int = 0
    m_group: int = 0
    per_row: bool = False

    def __post_init__(self):
        if self.kind == "unstructured":
            if not (0.0 <= self.sparsity <= 1.0):
                raise ValueError("sparsity must lie in [0, 1]")
        elif self.kind == "nm":
            if not (self.m_group >= 1 and 0 <= self.n_keep <= self.m_group):
                raise ValueError("N:M needs 0 <= N <= M and M >= 1")
        else:
            raise ValueError(f"unknown pattern kind {self.kind!r}")


def parse_pattern(p) -> Pattern:
    """``0.5`` -> 50% unstructured over each whole block; ``"0.5/row"`` -> 50%
    of every row of each block; ``"2:4"`` -> keep 2 of every 4."""
    if isinstance(p, Pattern):
        return p
    if isinstance(p, str) and ":" in p:
        a, b = p.split(":")
        return Pattern("nm", n_keep=int(a), m_group=int(b))
    if isinstance(p, str) and p.endswith("/row"):
        return Pattern("unstructured", sparsity=float(p[:-4]), per_row=True)
    return Pattern("unstructured", sparsity=float(p))


def unstructured_k(sparsity: float, rows: int, width: int) -> int:
    """Number of weights pruned in one column block of ``rows`` x ``width``.

    Reading (pages silent on rounding): floor(p * rows * width) evaluated in
    IEEE double exactly in this order, ((p * rows) * width).
    """
    return int(math.floor(sparsity * float(rows) * float(width)))


# ----------------------------------------------------------------------------
# a1: Hessian proxy
# ----------------------------------------------------------------------------

def hessian(x_chunks: Iterable[np.ndarray]) -> np.ndarray:
    """H = X X^T summed over all calibration tokens ([SGR] section 7, and
    section 10: calibration samples are used to estimate H = X X^T).

    Reading: the raw sum over tokens (no 1/N, no factor 2).  With token-major
    chunks Xc[t, c] this is sum_chunks Xc^T Xc.
    """
    H = None
    for xc in x_chunks:
        xd = np.asarray(xc, dtype=np.float64)
        part = xd.T @ xd
        H = part if H is None else H + part
    if H is None:
        raise ValueError("no calibration chunks")
    return H


# ----------------------------------------------------------------------------
# a2 + a3: damping and the inverse factor
# ----------------------------------------------------------------------------

def dampen(H: np.ndarray, damp: float):
    """H_d = H + lambda I with lambda = damp * mean(diag H).

    The pages do not mention damping.  Reading: a fraction ``damp`` >= 0 of the
    mean diagonal added to every diagonal entry.  The mean diagonal must be
    finite and positive (an all-zero or non-finite H is an error).
    Returns (H_d, lambda).
    """
    n = H.shape[0]
    if not (damp >= 0.0 and math.isfinite(damp)):
        raise ValueError("damp must be finite and >= 0")
    mean = float(np.trace(H)) / n
    if not math.isfinite(mean) or mean <= 0.0:
        raise np.linalg.LinAlgError("mean(diag H) is not finite and positive")
    lam = damp * mean
    return H + lam * np.eye(n), lam


def inverse_upper_factor(Hd: np.ndarray) -> np.ndarray:
    """U = the upper-triangular Cholesky factor of H_d^{-1} (H_d^{-1} = U^T U).

    The pages only say the error is estimated from the inverse Hessian ([SGR]
    section 8).  Textbook route, three library steps (LAPACK through PyTorch's
    CPU fp64 linear algebra): Cholesky of H_d, the inverse from that factor,
    Cholesky of the inverse, transposed to upper form.
    Row j of U satisfies U_jj * U[j, j:] = first row of (H_d[j:, j:])^{-1},
    i.e. it carries the inverse Hessian of the still-unprocessed columns.
    """
    Hd_t = torch.from_numpy(np.ascontiguousarray(Hd, dtype=np.float64))
    L = torch.linalg.cholesky(Hd_t)          # H_d = L L^T
    Hinv = torch.cholesky_inverse(L)         # H_d^{-1} from its Cholesky factor
    Hinv = 0.5 * (Hinv + Hinv.T)
    return torch.linalg.cholesky(Hinv).T.contiguous().numpy()


# ----------------------------------------------------------------------------
# a4 - a7: selection, OBS prune-and-compensate, finalize (unbatched)
# ----------------------------------------------------------------------------

def _select_block_unstructured(s: np.ndarray, row0_index: np.ndarray, k: int):
    """Boolean mask of the k smallest keys (s, linear index) of a block."""
    flat_s = s.ravel()
    flat_i = row0_index.ravel()
    order = np.lexsort((flat_i, flat_s))  # primary s, then index
    sel = np.zeros(flat_s.size, dtype=bool)
    sel[order[:k]] = True
    return sel.reshape(s.shape)


def _select_rows(s: np.ndarray, k: int):
    """Boolean mask of the k smallest keys (s, column) of every row."""
    order = np.argsort(s, axis=1, kind="stable")  # ties: lower column first
    sel = np.zeros(s.shape, dtype=bool)
    np.put_along_axis(sel, order[:, :k], True, axis=1)
    return sel


def prune(W: np.ndarray, U: np.ndarray, pattern, blocksize: int,
          mask_in: Optional[np.ndarray] = None, return_trace: bool = False):
    """Column-by-column OBS pruning with immediate (unbatched) compensation.

    [SGR] section 8: pick a weight, estimate the error of removing it from the
    inverse Hessian, set it to zero and update the other not-yet-pruned weights
    of the same row to compensate.  [SGR] section 11 steps 4-5 and [VSG] 02:
    columns are processed block by block in order, the chosen fraction is
    pruned and the rest updated, the error being passed on to later columns.

    Readings where the pages are silent:
      * saliency of weight (r, c) when it is chosen: Ŵ[r,c]^2 / U_cc^2, the
        OBS error of removing it with columns >= c still free;
      * compensation reaches only columns not yet processed (to the right);
      * unstructured: at each block start, prune exactly
        floor(p * m * w) weights of the whole m x w block, the smallest keys
        (saliency, r*n + c) in lexicographic order (lower index first on ties);
        per row (``"p/row"``): floor(p * w) weights of each row of the block,
        the smallest keys (saliency, c);
      * N:M: at each group start (column = 0 mod M), per row, prune the M-N
        smallest keys (saliency, c) of the group;
      * ``mask_in`` (m x n, True = prune) replaces selection;
      * a pruned weight is written as +0.0.

    Returns (W_hat, mask, eps) with eps[r] = sum of e^2 over row r's pruned
    weights, e = Ŵ[r,j] / U_jj at prune time.  With ``return_trace`` also a
    dict with the saliency of every weight at its selection point (computed
    along the actual trajectory also when ``mask_in`` forces the mask) and, per
    unstructured block, the k-th and (k+1)-th smallest saliency.
    """
    pat = parse_pattern(pattern)
    Wh = np.array(W, dtype=np.float64, copy=True)
    m, n = Wh.shape
    U = np.asarray(U, dtype=np.float64)
    if U.shape != (n, n):
        raise ValueError("U must be n x n")
    if blocksize < 1:
        raise ValueError("blocksize must be >= 1")
    if pat.kind == "nm" and n % pat.m_group != 0:
        raise ValueError("N:M needs M to divide n")
    mask = np.zeros((m, n), dtype=bool)
    eps = np.zeros(m, dtype=np.float64)
    d = np.diag(U).copy()
    sal = np.full((m, n), np.nan)
    block_thresholds = []
    lin = np.arange(m, dtype=np.int64)[:, None] * n

    for j in range(n):
        if pat.kind == "unstructured" and j % blocksize == 0:
            w = min(blocksize, n - j)
            s = Wh[:, j:j + w] ** 2 / d[j:j + w] ** 2
            sal[:, j:j + w] = s
            if mask_in is None and pat.per_row:
                mask[:, j:j + w] = _select_rows(s, unstructured_k(pat.sparsity, 1, w))
            elif mask_in is None:
                k = unstructured_k(pat.sparsity, m, w)
                idx = lin + np.arange(j, j + w, dtype=np.int64)[None, :]
                mask[:, j:j + w] = _select_block_unstructured(s, idx, k)
                ss = np.sort(s.ravel())
                kth = ss[k - 1] if k >= 1 else -np.inf
                nxt = ss[k] if k < ss.size else np.inf
                block_thresholds.append((j, w, k, kth, nxt))
        elif pat.kind == "nm" and j % pat.m_group == 0:
            M = pat.m_group
            s = Wh[:, j:j + M] ** 2 / d[j:j + M] ** 2
            sal[:, j:j + M] = s
            if mask_in is None:
                mask[:, j:j + M] = _select_rows(s, M - pat.n_keep)
        if mask_in is not None:
            mask[:, j] = np.asarray(mask_in[:, j], dtype=bool)

        rows = np.nonzero(mask[:, j])[0]
        if rows.size:
            e = Wh[rows, j] / U[j, j]
            Wh[rows, j:] -= np.outer(e, U[j, j:])
            Wh[rows, j] = 0.0
            eps[rows] += e * e

    if return_trace:
        return Wh, mask, eps, {"saliency": sal, "blocks": block_thresholds}
    return Wh, mask, eps


# ----------------------------------------------------------------------------
# Joint sparse + quantized sweep
# ----------------------------------------------------------------------------

def quant_grid(W: np.ndarray, bits: int):
    """Per-row uniform grid with 2^bits levels spanning the row's original
    weights and 0 (the pages name 4- and 8-bit weights but no grid).

    Reading: lo = min(0, min_j w_j), hi = max(0, max_j w_j),
    scale = (hi - lo) / (2^bits - 1) (1 for an all-zero row), integer zero
    point z = round(-lo / scale), rounding half to even throughout.  Returns
    (scale[m], zero[m]) as float64.
    """
    if not (2 <= bits <= 8):
        raise ValueError("bits must lie in [2, 8]")
    W = np.asarray(W, dtype=np.float64)
    lo = np.minimum(W.min(axis=1), 0.0)
    hi = np.maximum(W.max(axis=1), 0.0)
    levels = float(2 ** bits - 1)
    scale = np.where(hi > lo, (hi - lo) / levels, 1.0)
    zero = np.rint(-lo / scale)
    return scale, zero


def quant_code(x, scale, zero, bits: int):
    """Integer code of x on the grid: clamp(round(x / scale) + z, 0, 2^bits - 1)."""
    return np.clip(np.rint(x / scale) + zero, 0.0, float(2 ** bits - 1))


def prune_quantized(W: np.ndarray, U: np.ndarray, pattern, blocksize: int, bits: int,
                    mask_in: Optional[np.ndarray] = None,
                    codes_in: Optional[np.ndarray] = None, return_trace: bool = False):
    """Pruning and quantization in one column sweep ([SGR] section 15: the
    kept weights of a pruned layer can also be quantized to few bits;
    section 17: GPTQ quantizes weight by weight and compensates the rounding
    error through the inverse Hessian, the same second-order step SparseGPT
    uses for pruning).

    Same column order, selection points and saliencies as ``prune``.  At
    column j every row's weight is either pruned (target 0) or kept and
    rounded to its row's grid (target scale * (code - z)); in both cases
    e = (Ŵ[r,j] - target) / U_jj, the not-yet-processed weights of the row
    take Ŵ[r, j:] -= e * U[j, j:], and Ŵ[r,j] = target exactly.

    ``codes_in`` (m x n) replaces the rounding decisions (for comparisons
    along another implementation's trajectory).  Returns (W_hat, mask, eps,
    codes, scale, zero); codes of pruned weights are z (their value is 0).
    With ``return_trace`` also a dict with the saliency of every weight at
    its selection point, the value of every weight when it was quantized and
    the error e of every column step.
    """
    pat = parse_pattern(pattern)
    Wh = np.array(W, dtype=np.float64, copy=True)
    m, n = Wh.shape
    U = np.asarray(U, dtype=np.float64)
    if U.shape != (n, n):
        raise ValueError("U must be n x n")
    if pat.kind == "nm" and n % pat.m_group != 0:
        raise ValueError("N:M needs M to divide n")
    scale, zero = quant_grid(Wh, bits)
    mask = np.zeros((m, n), dtype=bool)
    codes = np.zeros((m, n), dtype=np.float64)
    eps = np.zeros(m)
    d = np.diag(U).copy()
    sal = np.full((m, n), np.nan)
    at_quant = np.full((m, n), np.nan)
    errs = np.zeros((m, n))
    lin = np.arange(m, dtype=np.int64)[:, None] * n

    for j in range(n):
        if pat.kind == "unstructured" and j % blocksize == 0:
            w = min(blocksize, n - j)
            s = Wh[:, j:j + w] ** 2 / d[j:j + w] ** 2
            sal[:, j:j + w] = s
            if mask_in is None and pat.per_row:
                mask[:, j:j + w] = _select_rows(s, unstructured_k(pat.sparsity, 1, w))
            elif mask_in is None:
                idx = lin + np.arange(j, j + w, dtype=np.int64)[None, :]
                mask[:, j:j + w] = _select_block_unstructured(s, idx, unstructured_k(pat.sparsity, m, w))
        elif pat.kind == "nm" and j % pat.m_group == 0:
            M = pat.m_group
            s = Wh[:, j:j + M] ** 2 / d[j:j + M] ** 2
            sal[:, j:j + M] = s
            if mask_in is None:
                mask[:, j:j + M] = _select_rows(s, M - pat.n_keep)
        if mask_in is not None:
            mask[:, j] = np.asarray(mask_in[:, j], dtype=bool)

        x = Wh[:, j].copy()
        at_quant[:, j] = x
        if codes_in is not None:
            c = np.asarray(codes_in[:, j], dtype=np.float64)
        else:
            c = quant_code(x, scale, zero, bits)
        c = np.where(mask[:, j], zero, c)
        target = scale * (c - zero)
        e = (x - target) / U[j, j]
        Wh[:, j:] -= np.outer(e, U[j, j:])
        Wh[:, j] = np.where(mask[:, j], 0.0, target)
        codes[:, j] = c
        errs[:, j] = e
        eps += e * e

    out = (Wh, mask, eps, codes.astype(np.uint8), scale, zero)
    if return_trace:
        return out + ({"saliency": sal, "at_quant": at_quant, "errors": errs},)
    return out


# ----------------------------------------------------------------------------
# Vector-level joint compensation
# ----------------------------------------------------------------------------

def prune_vector(W: np.ndarray, U: np.ndarray, pattern, blocksize: int, vec: int,
                 mask_in: Optional[np.ndarray] = None, return_trace: bool = False):
    """Joint (vector-level) removal of the chosen weights of each range of
    ``vec`` consecutive columns ([VSG] 01-02: instead of removing weights one
    after another and compensating after each, the weights chosen within a
    range are set to zero together and the kept weights are adjusted jointly;
    the matrix is processed in smaller units whose error is passed on to the
    later parts).

    The pages give no formula.  Readings:
      * ranges are [j0, j0 + vec) for j0 = 0, vec, 2 vec, ...; vec divides
        the block size (and, under N:M, M divides vec or vec divides M);
        vec = 1 is the column-by-column procedure of ``prune``;
      * selection rules, counts and saliencies are those of ``prune``; a
        selection point inside a range sees the values at the range start
        (nothing changes inside a range before its joint step);
      * at each range start every row with a non-empty chosen set P in the
        range removes it at once with the exact multi-weight OBS update over
        the free columns F = [j0, n):  with G = (H_d[F,F])^-1 = U_FF^T U_FF,
        delta_F = -w_P (G_PP)^-1 G_P,F,  then w_P = +0.0; earlier columns
        stay frozen.  Its damped error is w_P (G_PP)^-1 w_P^T.

    Returns (W_hat, mask, eps); with ``return_trace`` also a dict holding the
    saliencies at selection and the per-range error rows e (w - w_hat =
    e U, e supported on each range's rows of U).
    """
    pat = parse_pattern(pattern)
    Wh = np.array(W, dtype=np.float64, copy=True)
    m, n = Wh.shape
    U = np.asarray(U, dtype=np.float64)
    if U.shape != (n, n):
        raise ValueError("U must be n x n")
    if vec < 1 or blocksize % vec != 0:
        raise ValueError("vec must divide the block size")
    if pat.kind == "nm":
        if n % pat.m_group != 0:
            raise ValueError("N:M needs M to divide n")
        if vec % pat.m_group != 0 and pat.m_group % vec != 0:
            raise ValueError("N:M needs M | vec or vec | M")
    mask = np.zeros((m, n), dtype=bool)
    eps = np.zeros(m)
    d = np.diag(U).copy()
    sal = np.full((m, n), np.nan)
    errs = np.zeros((m, n))
    lin = np.arange(m, dtype=np.int64)[:, None] * n

    for j0 in range(0, n, vec):
        j1 = min(n, j0 + vec)
        for j in range(j0, j1):
            if pat.kind == "unstructured" and j % blocksize == 0:
                w = min(blocksize, n - j)
                s = Wh[:, j:j + w] ** 2 / d[j:j + w] ** 2
                sal[:, j:j + w] = s
                if mask_in is None and pat.per_row:
                    mask[:, j:j + w] = _select_rows(s, unstructured_k(pat.sparsity, 1, w))
                elif mask_in is None:
                    idx = lin + np.arange(j, j + w, dtype=np.int64)[None, :]
                    mask[:, j:j + w] = _select_block_unstructured(s, idx, unstructured_k(pat.sparsity, m, w))
            elif pat.kind == "nm" and j % pat.m_group == 0:
                M = pat.m_group
                s = Wh[:, j:j + M] ** 2 / d[j:j + M] ** 2
                sal[:, j:j + M] = s
                if mask_in is None:
                    mask[:, j:j + M] = _select_rows(s, M - pat.n_keep)
        if mask_in is not None:
            mask[:, j0:j1] = np.asarray(mask_in[:, j0:j1], dtype=bool)

        UF = U[j0:, j0:]
        for r in range(m):
            Pl = np.nonzero(mask[r, j0:j1])[0]
            if Pl.size == 0:
                continue
            A = UF[:, Pl]                      # U_F,P
            G_PP = A.T @ A
            G_PF = A.T @ UF
            wP = Wh[r, j0 + Pl].copy()
            y = np.linalg.solve(G_PP, wP)
            Wh[r, j0:] -= y @ G_PF
            Wh[r, j0 + Pl] = 0.0
            eps[r] += float(y @ wP)
            errs[r, j0:j1] = (A @ y)[:j1 - j0]

    if return_trace:
        return Wh, mask, eps, {"saliency": sal, "errors": errs}
    return Wh, mask, eps


def prune_free_set(W: np.ndarray, Hd: np.ndarray, pattern, blocksize: int,
                   mask_in: Optional[np.ndarray] = None):
    """The same procedure without any Cholesky factor (cross-check route).

    Keeps G = (H_d[F, F])^{-1} for the free set F = {j, ..., n-1} and removes
    column j from it by the elimination downdate G <- G - G[:,0] G[0,:]/G_00
    after each step.  The OBS quantities are read from G directly: the error of
    removing w_j is w_j^2 / G_00 and the compensation of the free weights is
    -(w_j / G_00) * G[0, :] ([SGR] section 8).  Intended for n <= ~1024.
    """
    pat = parse_pattern(pattern)
    Wh = np.array(W, dtype=np.float64, copy=True)
    m, n = Wh.shape
    G = np.linalg.inv(np.asarray(Hd, dtype=np.float64))
    mask = np.zeros((m, n), dtype=bool)
    eps = np.zeros(m)
    lin = np.arange(m, dtype=np.int64)[:, None] * n
    def downdate(Gj):
        return Gj[1:, 1:] - np.outer(Gj[1:, 0], Gj[0, 1:]) / Gj[0, 0]

    diag_at = np.zeros(n)  # G_00 of the free set that starts at column j
    Gj = G.copy()
    for j in range(n):
        diag_at[j] = Gj[0, 0]
        if j + 1 < n:
            Gj = downdate(Gj)

    Gj = G.copy()
    for j in range(n):
        if j > 0:
            Gj = downdate(Gj)
        if mask_in is not None:
            mask[:, j] = np.asarray(mask_in[:, j], dtype=bool)
        elif pat.kind == "unstructured" and j % blocksize == 0:
            w = min(blocksize, n - j)
            s = Wh[:, j:j + w] ** 2 / diag_at[j:j + w]
            if pat.per_row:
                mask[:, j:j + w] = _select_rows(s, unstructured_k(pat.sparsity, 1, w))
            else:
                k = unstructured_k(pat.sparsity, m, w)
                idx = lin + np.arange(j, j + w, dtype=np.int64)[None, :]
                mask[:, j:j + w] = _select_block_unstructured(s, idx, k)
        elif pat.kind == "nm" and j % pat.m_group == 0:
            M = pat.m_group
            s = Wh[:, j:j + M] ** 2 / diag_at[j:j + M]
            mask[:, j:j + M] = _select_rows(s, M - pat.n_keep)
        rows = np.nonzero(mask[:, j])[0]
        if rows.size:
            wq = Wh[rows, j]
            Wh[rows, j:] -= np.outer(wq / Gj[0, 0], Gj[0, :])
            Wh[rows, j] = 0.0
            eps[rows] += wq * wq / Gj[0, 0]
    return Wh, mask, eps


# ----------------------------------------------------------------------------
# a8: reconstruction error
# ----------------------------------------------------------------------------

def reconstruction_error(W: np.ndarray, W_hat: np.ndarray,
                         x_chunks: Iterable[np.ndarray]) -> float:
    """E = ||W X - Ŵ X||_F^2 summed over all tokens ([SGR] section 6: keep Ŵ X
    as close as possible to W X).  W is the original (undamped problem)."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    E = 0.0
    for xc in x_chunks:
        Y = D @ np.asarray(xc, dtype=np.float64).T
        E += float(np.sum(Y * Y))
    return E


def reconstruction_error_from_hessian(W, W_hat, H) -> float:
    """Same quantity through H: sum over rows of d H d^T with d = w - ŵ."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    return float(np.sum((D @ np.asarray(H, dtype=np.float64)) * D))


# ----------------------------------------------------------------------------
# 2:4 compressed export
# ----------------------------------------------------------------------------

def pack_two_four(W_hat: np.ndarray, mask: np.ndarray):
    """The 2:4 compressed form of a pruned matrix: the kept values plus a
    2-bit position index per kept value ([G24] 2:4 core-mechanism section: two
    of every four consecutive values along the reduction axis are kept and
    their positions are recorded in 2-bit metadata).

    Readings (the page fixes no byte layout):
      * group g of row r = columns 4g .. 4g+3; its two slots hold the kept
        positions in increasing order; a group with fewer than two kept
        positions fills the remaining slots with its lowest pruned positions
        (value +0.0), so the slot indices are always two distinct positions
        i0 < i1;
      * values[r, 2g + s] = W_hat at slot s (0.0 for a pruned slot);
      * meta[r, g // 2] holds group g in its low nibble (g even) or high nibble
        (g odd); the nibble is i0 | (i1 << 2);
      * a group with more than two kept positions cannot be represented: it
        is counted in ``bad`` and its two lowest kept positions are stored.

    Returns (values [m, n/2] float64, meta [m, ceil(n/8)] uint8, bad).
    """
    W_hat = np.asarray(W_hat, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    m, n = W_hat.shape
    if n % 4 != 0:
        raise ValueError("2:4 export needs 4 | n")
    ng = n // 4
    values = np.zeros((m, 2 * ng), dtype=np.float64)
    meta = np.zeros((m, (ng + 1) // 2), dtype=np.uint8)
    bad = 0
    for r in range(m):
        for g in range(ng):
            kept = [i for i in range(4) if not mask[r, 4 * g + i]]
            pruned = [i for i in range(4) if mask[r, 4 * g + i]]
            if len(kept) > 2:
                bad += 1
            i0, i1 = sorted((kept + pruned)[:2])
            for slot, i in enumerate((i0, i1)):
                if not mask[r, 4 * g + i]:
                    values[r, 2 * g + slot] = W_hat[r, 4 * g + i]
            meta[r, g // 2] |= (i0 | (i1 << 2)) << (4 * (g % 2))
    return values, meta, bad


def unpack_two_four(values: np.ndarray, meta: np.ndarray, n: int) -> np.ndarray:
    """Dense m x n matrix from its 2:4 compressed form (inverse of
    pack_two_four for masks with at most two kept positions per group)."""
    values = np.asarray(values, dtype=np.float64)
    m = values.shape[0]
    out = np.zeros((m, n), dtype=np.float64)
    for r in range(m):
        for g in range(n // 4):
            nib = (int(meta[r, g // 2]) >> (4 * (g % 2))) & 0xF
            out[r, 4 * g + (nib & 3)] = values[r, 2 * g]
            out[r, 4 * g + (nib >> 2)] = values[r, 2 * g + 1]
    return out


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def solve_layer(W, x_chunks, pattern, blocksize: int, damp: float = 0.01,
                mask_in=None):
    """a1 .. a7 in order ([SGR] section 11 steps 3-5) for one linear layer.

    Returns a dict with H, lambda, U, W_hat, mask, eps and E (the
    reconstruction error of Ŵ over the same chunks).
    """
    chunks = list(x_chunks)
    H = hessian(chunks)
    Hd, lam = dampen(H, damp)
    U = inverse_upper_factor(Hd)
    Wh, mask, eps = prune(W, U, pattern, blocksize, mask_in=mask_in)
    E = reconstruction_error(W, Wh, chunks)
    return {"H": H, "lam": lam, "U": U, "W_hat": Wh, "mask": mask,
            "eps": eps, "E": E}
