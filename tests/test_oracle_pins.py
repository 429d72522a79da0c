"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only.  Each test checks the oracle against something other than itself: a
brute-force loop, a closed form, a textbook least-squares solution, an
exhaustive search, a printed worked example, or an invariance of the method.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import Pattern

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng


def _spd_inputs(seed, n, tokens, corr=0.6):
    r = rng0(seed)
    A = np.eye(n) + corr * r.standard_normal((n, n)) / math.sqrt(n)
    s = np.exp(r.standard_normal(n))
    return (r.standard_normal((tokens, n)) @ A) * s[None, :]


def _layer(seed, m, n, tokens, damp=0.01):
    X = _spd_inputs(seed, n, tokens)
    W = rng0(seed + 1).standard_normal((m, n)) * 0.02
    H = oracle.hessian([X])
    Hd, lam = oracle.dampen(H, damp)
    U = oracle.inverse_upper_factor(Hd)
    return W, X, H, Hd, lam, U


def _quad(d, Hd):
    return float(d @ Hd @ d)


# ----------------------------------------------------------------------------
# a1 Hessian
# ----------------------------------------------------------------------------

def test_hessian_brute_force_loops():
    r = rng0(1)
    X = r.standard_normal((7, 5))
    H = oracle.hessian([X[:3], X[3:]])
    for i in range(5):
        for j in range(5):
            acc = 0.0
            for t in range(7):
                acc += X[t, i] * X[t, j]
            assert abs(H[i, j] - acc) <= 1e-13 * max(1.0, abs(acc))


def test_hessian_orthogonal_columns_closed_form():
    # Columns of a 8x8 Hadamard matrix are orthogonal with squared norm 8.
    Hd8 = np.array([[1]])
    for _ in range(3):
        Hd8 = np.block([[Hd8, Hd8], [Hd8, -Hd8]])
    scales = np.array([1.0, 2.0, 0.5, 3.0, 1.5, 0.25, 4.0, 1.0])
    X = Hd8 * scales[None, :]
    H = oracle.hessian([X])
    assert np.array_equal(H, np.diag(8.0 * scales ** 2))


def test_hessian_symmetric_psd_and_chunk_additive():
    X = _spd_inputs(3, 24, 200)
    H = oracle.hessian([X])
    H2 = oracle.hessian([X[:17], X[17:101], X[101:]])
    assert np.allclose(H, H.T, rtol=0, atol=0)
    assert np.allclose(H, H2, rtol=1e-13, atol=1e-12)
    assert np.linalg.eigvalsh(H).min() > -1e-9


# ----------------------------------------------------------------------------
# a2/a3 damping and the inverse factor U
# ----------------------------------------------------------------------------

def test_damping_closed_form():
    H = np.diag([1.0, 2.0, 3.0, 6.0])
    Hd, lam = oracle.dampen(H, 0.01)
    assert lam == pytest.approx(0.01 * 3.0)
    assert np.allclose(Hd, np.diag([1.03, 2.03, 3.03, 6.03]))
    with pytest.raises(np.linalg.LinAlgError):
        oracle.dampen(np.zeros((3, 3)), 0.01)


def test_inverse_factor_2x2_closed_form():
    a, b, c = 3.0, 1.2, 2.0
    det = a * c - b * b
    U = oracle.inverse_upper_factor(np.array([[a, b], [b, c]]))
    assert U[1, 0] == 0.0
    assert U[0, 0] == pytest.approx(math.sqrt(c / det), rel=1e-14)
    assert U[0, 1] == pytest.approx(-b / math.sqrt(c * det), rel=1e-14)
    assert U[1, 1] == pytest.approx(1.0 / math.sqrt(c), rel=1e-14)


def test_inverse_factor_diagonal():
    h = np.array([0.5, 2.0, 9.0, 1.0, 4.0])
    U = oracle.inverse_upper_factor(np.diag(h))
    assert np.allclose(U, np.diag(1.0 / np.sqrt(h)), rtol=1e-15, atol=0)


def test_inverse_factor_identities():
    _, _, _, Hd, _, U = _layer(5, 4, 40, 300)
    n = Hd.shape[0]
    assert np.all(np.tril(U, -1) == 0.0)
    assert np.all(np.diag(U) > 0)
    assert np.abs(U.T @ U @ Hd - np.eye(n)).max() < 1e-10
    for j in (0, 1, 7, 23, n - 2, n - 1):
        Gj = np.linalg.inv(Hd[j:, j:])
        assert U[j, j] ** 2 == pytest.approx(Gj[0, 0], rel=1e-11)
        assert np.allclose(U[j, j] * U[j, j:], Gj[0, :], rtol=1e-10, atol=1e-13)
    # trailing block of U depends only on the trailing block of H_d
    s = 25
    Us = oracle.inverse_upper_factor(Hd[s:, s:])
    assert np.allclose(U[s:, s:], Us, rtol=1e-10, atol=1e-13)


# ----------------------------------------------------------------------------
# a4-a7 OBS prune and compensate
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("q", [0, 5, 11])
def test_single_weight_obs_closed_form(q):
    W, _, _, Hd, _, U = _layer(7, 3, 12, 80)
    n = W.shape[1]
    mask = np.zeros_like(W, dtype=bool)
    mask[:, q] = True
    Wh, M, eps = oracle.prune(W, U, 0.0, 4, mask_in=mask)
    F = np.arange(q, n)
    G = np.linalg.inv(Hd[np.ix_(F, F)])
    for r in range(W.shape[0]):
        wq = W[r, q]
        delta = -wq / G[0, 0] * G[:, 0]
        expect = W[r].copy()
        expect[F] += delta
        assert np.allclose(Wh[r], expect, rtol=0, atol=1e-14)
        assert Wh[r, q] == 0.0 and not np.signbit(Wh[r, q])
        assert np.array_equal(Wh[r, :q], W[r, :q])
        assert eps[r] == pytest.approx(wq * wq / G[0, 0], rel=1e-12)


def test_prefix_mask_is_least_squares_optimum():
    W, _, _, Hd, _, U = _layer(8, 4, 16, 120)
    k = 6
    mask = np.zeros_like(W, dtype=bool)
    mask[:, :k] = True
    Wh, _, _ = oracle.prune(W, U, 0.0, 8, mask_in=mask)
    K = np.arange(k, W.shape[1])
    for r in range(W.shape[0]):
        wK = np.linalg.solve(Hd[np.ix_(K, K)], Hd[K, :] @ W[r])
        assert np.allclose(Wh[r, K], wK, rtol=1e-10, atol=1e-13)
        assert np.all(Wh[r, :k] == 0.0)


def _sequential_error_bruteforce(w, Hd, q):
    """Error of removing only weight q with the frozen prefix / free suffix
    convention: minimise (w - v) H_d (w - v)^T over v with v[:q] = w[:q],
    v[q] = 0 and v[q+1:] free, by an explicit normal-equation solve."""
    n = w.size
    free = np.arange(q + 1, n)
    fixed_d = np.zeros(n)
    fixed_d[q] = w[q]                       # d = w - v on the fixed part
    if free.size:
        rhs = -(Hd[np.ix_(free, [q])] @ np.array([w[q]]))
        d_free = np.linalg.solve(Hd[np.ix_(free, free)], rhs)
        fixed_d[free] = d_free
    return _quad(fixed_d, Hd)


def test_exhaustive_single_weight_choice_n8():
    # k = 1 of an 8-input row in one block: the oracle's pick is the argmin of
    # the true sequential error over all 8 candidates.
    hits = 0
    for t in range(60):
        W, _, _, Hd, _, U = _layer(100 + t, 1, 8, 40)
        Wh, M, eps = oracle.prune(W, U, 1.0 / 8.0, 8)
        assert M.sum() == 1
        errs = [_sequential_error_bruteforce(W[0], Hd, q) for q in range(8)]
        assert int(np.nonzero(M[0])[0][0]) == int(np.argmin(errs))
        assert eps[0] == pytest.approx(min(errs), rel=1e-9)
        hits += 1
    assert hits == 60


def test_error_identity_any_mask_and_ls_bound_n8():
    # (iii) for any mask the damped error equals the sum of e^2;
    # (ii) the greedy result is never below the exhaustive LS optimum.
    for t in range(25):
        W, _, _, Hd, _, U = _layer(300 + t, 1, 8, 40)
        w = W[0]
        r = rng0(t)
        mask = np.zeros((1, 8), dtype=bool)
        mask[0, r.choice(8, 3, replace=False)] = True
        Wh, _, eps = oracle.prune(W, U, 0.0, 8, mask_in=mask)
        d = w - Wh[0]
        assert _quad(d, Hd) == pytest.approx(eps[0], rel=1e-10)

        Wg, Mg, eg = oracle.prune(W, U, 0.5, 8)
        k = int(Mg.sum())
        assert k == 4
        best = np.inf
        for P in itertools.combinations(range(8), k):
            P = list(P)
            K = [c for c in range(8) if c not in P]
            vK = np.linalg.solve(Hd[np.ix_(K, K)], Hd[K, :] @ w)
            v = np.zeros(8)
            v[K] = vK
            best = min(best, _quad(w - v, Hd))
        assert eg[0] >= best * (1 - 1e-12)


def test_unstructured_counts_ragged_and_exact_zeros():
    W, _, _, _, _, U = _layer(11, 13, 50, 200)
    B, p = 16, 0.55
    Wh, M, _ = oracle.prune(W, U, p, B)
    m, n = W.shape
    for j in range(0, n, B):
        w = min(B, n - j)
        assert M[:, j:j + w].sum() == math.floor(p * m * w)
    assert np.all(Wh[M] == 0.0) and not np.any(np.signbit(Wh[M]))
    assert np.all(Wh[~M] != 0.0)


# ----------------------------------------------------------------------------
# a4 per-row unstructured granularity
# ----------------------------------------------------------------------------

def test_per_row_counts_ragged_and_exact_zeros():
    W, _, _, _, _, U = _layer(31, 11, 50, 200)
    B, p = 16, 0.55
    Wh, M, _ = oracle.prune(W, U, f"{p}/row", B)
    for j in range(0, W.shape[1], B):
        w = min(B, W.shape[1] - j)
        assert np.all(M[:, j:j + w].sum(axis=1) == math.floor(p * w))
    assert np.all(Wh[M] == 0.0) and not np.any(np.signbit(Wh[M]))


def test_per_row_identity_hessian_is_row_magnitude_pruning():
    # H proportional to I: saliency is w^2 times a constant and nothing is
    # compensated, so each row of each block drops its floor(p w) smallest
    # magnitudes (lower column first on ties); brute force per row.
    r = rng0(32)
    W = np.round(r.standard_normal((5, 37)), 1)  # rounding creates ties
    Hd, _ = oracle.dampen(2.0 * np.eye(37), 0.01)
    U = oracle.inverse_upper_factor(Hd)
    B, p = 12, 0.4
    Wh, M, _ = oracle.prune(W, U, f"{p}/row", B)
    for j in range(0, 37, B):
        w = min(B, 37 - j)
        k = math.floor(p * w)
        for row in range(5):
            keyed = sorted((abs(W[row, j + c]), c) for c in range(w))
            want = np.zeros(w, dtype=bool)
            for _, c in keyed[:k]:
                want[c] = True
            assert np.array_equal(M[row, j:j + w], want)
    assert np.array_equal(Wh[~M], W[~M])


def test_per_row_exhaustive_single_weight_choice_n8():
    # one pruned weight per row of an 8-wide block: each row's pick is the
    # argmin over its 8 single-weight masks of the exact damped error
    # min_v (w - v) H_d (w - v)^T with v_q = 0 (textbook least squares)
    W, _, _, Hd, _, U = _layer(33, 6, 8, 60)
    _, M, _ = oracle.prune(W, U, "0.125/row", 8)
    for row in range(6):
        w = W[row]
        errs = []
        for q in range(8):
            K = [c for c in range(8) if c != q]
            v = np.zeros(8)
            v[K] = np.linalg.solve(Hd[np.ix_(K, K)], Hd[K, :] @ w)
            errs.append(_quad(w - v, Hd))
        assert M[row].sum() == 1 and int(np.argmax(M[row])) == int(np.argmin(errs))


def test_per_row_rows_independent_and_one_row_equals_block_global():
    W, _, _, _, _, U = _layer(34, 7, 40, 150)
    Wa, Ma, _ = oracle.prune(W, U, "0.6/row", 16)
    for row in range(7):
        Wb, Mb, _ = oracle.prune(W[row:row + 1], U, "0.6/row", 16)
        Wc, Mc, _ = oracle.prune(W[row:row + 1], U, 0.6, 16)
        assert np.array_equal(Ma[row], Mb[0]) and np.array_equal(Wa[row], Wb[0])
        assert np.array_equal(Mb, Mc) and np.array_equal(Wb, Wc)


def test_per_row_with_block_m_equals_nm():
    # keeping N of every M per row with B = M is the per-row rule with
    # p = (M - N) / M (exact in binary for these fractions)
    W, _, _, _, _, U = _layer(35, 6, 64, 200)
    for N, M in ((2, 4), (16, 64), (4, 8)):
        a = oracle.prune(W, U, f"{N}:{M}", M)
        b = oracle.prune(W, U, f"{(M - N) / M}/row", M)
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])


# ----------------------------------------------------------------------------
# joint sparse + quantized sweep
# ----------------------------------------------------------------------------

def test_quant_grid_hand_examples():
    # worked by hand: [-1, 0.5, 2] at 2 bits spans [-1, 2]: scale 1, zero 1;
    # 0.5 / 1 is a tie that rounds to the even 0 -> code 1 -> value 0.
    # [0.25, 0.75, 1.75] at 3 bits spans [0, 1.75]: scale 0.25, zero 0.
    # [-0.5, 0.25, 1.0] at 2 bits spans [-0.5, 1]: scale 0.5, zero 1; 0.25 /
    # 0.5 = 0.5 ties to 0 -> code 1 -> value 0.
    for row, bits, sc, z, codes in (([-1.0, 0.5, 2.0], 2, 1.0, 1.0, [0, 1, 3]),
                                    ([0.25, 0.75, 1.75], 3, 0.25, 0.0, [1, 3, 7]),
                                    ([-0.5, 0.25, 1.0], 2, 0.5, 1.0, [0, 1, 3])):
        W = np.array([row])
        scale, zero = oracle.quant_grid(W, bits)
        assert scale[0] == sc and zero[0] == z
        got = oracle.quant_code(W[0], scale[0], zero[0], bits)
        assert list(got) == codes


def _nearest_level(x, scale, zero, bits):
    # brute force over all 2^bits levels; ties go to the even offset code - z
    best = None
    for c in range(2 ** bits):
        v = scale * (c - zero)
        key = (abs(x - v), (c - zero) % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_quantized_sweep_identity_hessian_is_round_to_nearest():
    # H ~ I: no compensation reaches other columns, so every kept weight is
    # simply its nearest grid level and the mask is magnitude pruning
    r = rng0(41)
    W = r.standard_normal((4, 24))
    Hd, _ = oracle.dampen(5.0 * np.eye(24), 0.01)
    U = oracle.inverse_upper_factor(Hd)
    for pat in (0.0, 0.5, "2:4"):
        Wh, M, _, C, scale, zero = oracle.prune_quantized(W, U, pat, 8, 3)
        _, Mp, _ = oracle.prune(W, U, pat, 8)
        assert np.array_equal(M, Mp)
        for i in range(4):
            for j in range(24):
                if M[i, j]:
                    assert Wh[i, j] == 0.0 and C[i, j] == zero[i]
                else:
                    c = _nearest_level(W[i, j], scale[i], zero[i], 3)
                    assert C[i, j] == c
                    assert Wh[i, j] == pytest.approx(scale[i] * (c - zero[i]), abs=1e-15)


def test_quantized_sweep_prefix_values_are_least_squares():
    # the value a weight has when it is quantized equals the textbook
    # constrained least-squares optimum with every earlier column fixed at
    # its final value: v_K = w_K + H_KK^-1 H_KP (w_P - t_P)
    W, _, _, Hd, _, U = _layer(42, 3, 20, 120)
    Wh, M, eps, C, _, _, tr = oracle.prune_quantized(W, U, 0.3, 5, 4, return_trace=True)
    for j in (1, 6, 13, 19):
        P = list(range(j))
        K = list(range(j, 20))
        for i in range(3):
            vK = W[i, K] + np.linalg.solve(Hd[np.ix_(K, K)], Hd[np.ix_(K, P)] @ (W[i, P] - Wh[i, P]))
            assert tr["at_quant"][i, j] == pytest.approx(vK[0], rel=1e-9, abs=1e-12)


def test_quantized_sweep_error_structure():
    # w - w_hat = e U row by row (each step moves the row along U's row j),
    # and the damped error equals the sum of e^2
    W, _, _, Hd, _, U = _layer(43, 5, 32, 150)
    for pat in (0.5, "4:8", "0.5/row"):
        Wh, M, eps, C, scale, zero, tr = oracle.prune_quantized(W, U, pat, 10, 3, return_trace=True)
        d = W - Wh
        assert np.abs(d - tr["errors"] @ U).max() < 1e-12
        for i in range(5):
            assert _quad(d[i], Hd) == pytest.approx(eps[i], rel=1e-9)
        # every value is on its row's grid, pruned ones exactly +0.0
        assert np.allclose(Wh, scale[:, None] * (C.astype(float) - zero[:, None]), atol=1e-15)
        assert np.all(Wh[M] == 0.0) and not np.any(np.signbit(Wh[M]))


def test_quantized_sweep_forced_decisions_reproduce():
    W, _, _, _, _, U = _layer(44, 4, 16, 80)
    a = oracle.prune_quantized(W, U, "2:4", 8, 4)
    b = oracle.prune_quantized(W, U, "2:4", 8, 4, mask_in=a[1], codes_in=a[3])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[3], b[3])


# ----------------------------------------------------------------------------
# vector-level joint compensation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pat", [0.5, "0.5/row", "2:4"])
def test_vector_range_one_is_column_by_column(pat):
    W, _, _, _, _, U = _layer(51, 6, 32, 150)
    a = oracle.prune(W, U, pat, 8)
    b = oracle.prune_vector(W, U, pat, 8, 1)
    assert np.array_equal(a[1], b[1])
    assert np.abs(a[0] - b[0]).max() < 1e-12
    assert np.allclose(a[2], b[2], rtol=1e-10)


def test_vector_single_range_is_least_squares_optimum():
    # one block, one range: the result is the textbook constrained least
    # squares optimum v_K = H_KK^-1 H_K,: w for the chosen mask, from H_d
    W, _, _, Hd, _, U = _layer(52, 5, 16, 100)
    Wh, M, eps = oracle.prune_vector(W, U, 0.5, 16, 16)
    for r in range(5):
        K = np.nonzero(~M[r])[0]
        v = np.zeros(16)
        v[K] = np.linalg.solve(Hd[np.ix_(K, K)], Hd[K, :] @ W[r])
        assert np.abs(Wh[r] - v).max() < 1e-10
        assert _quad(W[r] - v, Hd) == pytest.approx(eps[r], rel=1e-9)
    # and it is never worse than removing the same weights one at a time
    _, _, eps_seq = oracle.prune(W, U, 0.5, 16, mask_in=M)
    assert np.all(eps <= eps_seq * (1 + 1e-12))


def test_vector_last_range_is_least_squares_given_prefix():
    # after the last range's joint step nothing changes any more: its kept
    # weights are the least-squares optimum with every earlier column fixed at
    # its final value and the range's chosen weights at zero
    W, _, _, Hd, _, U = _layer(53, 4, 32, 160)
    Wh, M, _ = oracle.prune_vector(W, U, "0.5/row", 16, 8)
    j0 = 24
    for r in range(4):
        Q = list(range(j0)) + [j for j in range(j0, 32) if M[r, j]]
        K = [j for j in range(j0, 32) if not M[r, j]]
        t = np.where(M[r], 0.0, Wh[r])[Q]
        vK = W[r, K] + np.linalg.solve(Hd[np.ix_(K, K)], Hd[np.ix_(K, Q)] @ (W[r, Q] - t))
        assert np.abs(Wh[r, K] - vK).max() < 1e-10


@pytest.mark.parametrize("pat,vec", [(0.5, 8), ("4:8", 16), ("16:32", 16), ("0.6/row", 4)])
def test_vector_error_structure(pat, vec):
    W, _, _, Hd, _, U = _layer(54, 5, 64, 200)
    Wh, M, eps, tr = oracle.prune_vector(W, U, pat, 16, vec, return_trace=True)
    d = W - Wh
    assert np.abs(d - tr["errors"] @ U).max() < 1e-12
    for r in range(5):
        assert _quad(d[r], Hd) == pytest.approx(eps[r], rel=1e-9)
    assert np.all(Wh[M] == 0.0) and not np.any(np.signbit(Wh[M]))
    _, Mp, _ = oracle.prune(W, U, pat, 16)
    if vec == 1:
        assert np.array_equal(M, Mp)


def test_vector_prefix_masks_equal_column_by_column():
    # chosen sets that are prefixes of each range: removing them one at a time
    # with the later columns free is already the joint optimum
    W, _, _, _, _, U = _layer(55, 6, 32, 150)
    r = rng0(5)
    M = np.zeros((6, 32), dtype=bool)
    for i in range(6):
        for j0 in range(0, 32, 8):
            M[i, j0:j0 + int(r.integers(0, 9))] = True
    a = oracle.prune(W, U, 0.5, 8, mask_in=M)
    b = oracle.prune_vector(W, U, 0.5, 8, 8, mask_in=M)
    assert np.abs(a[0] - b[0]).max() < 1e-12


# ----------------------------------------------------------------------------
# 2:4 compressed export
# ----------------------------------------------------------------------------

def test_two_four_pack_golden():
    with open(os.path.join(GOLDEN, "two_four_packed.json")) as f:
        fx = json.load(f)
    for row in fx["rows"]:
        dense = np.array([row["dense"]])
        pruned = np.array([row["pruned"]], dtype=bool)
        Wh = np.where(pruned, 0.0, dense)
        vals, meta, bad = oracle.pack_two_four(Wh, pruned)
        assert bad == 0
        assert np.array_equal(vals[0], np.array(row["values"]))
        assert list(meta[0]) == row["meta"]


def test_two_four_pack_of_pruned_layer_round_trips():
    W, _, _, _, _, U = _layer(36, 9, 48, 200)
    Wh, M, _ = oracle.prune(W, U, "2:4", 16)
    vals, meta, bad = oracle.pack_two_four(Wh, M)
    assert bad == 0 and vals.shape == (9, 24) and meta.shape == (9, 6)
    assert np.array_equal(oracle.unpack_two_four(vals, meta, 48), Wh)
    # every slot index is a kept position, in increasing order
    for r in range(9):
        for g in range(12):
            nib = (int(meta[r, g // 2]) >> (4 * (g % 2))) & 0xF
            i0, i1 = nib & 3, nib >> 2
            assert i0 < i1 and not M[r, 4 * g + i0] and not M[r, 4 * g + i1]
            assert vals[r, 2 * g] == Wh[r, 4 * g + i0] and vals[r, 2 * g + 1] == Wh[r, 4 * g + i1]


def test_two_four_pack_sparse_groups_and_unrepresentable_count():
    r = rng0(37)
    m, n = 6, 40
    Wd = r.standard_normal((m, n))
    # per group: 0..4 pruned positions chosen at random
    M = np.zeros((m, n), dtype=bool)
    want_bad = 0
    for row in range(m):
        for g in range(n // 4):
            k = int(r.integers(0, 5))
            M[row, 4 * g + r.permutation(4)[:k]] = True
            want_bad += int(4 - k > 2)
    Wh = np.where(M, 0.0, Wd)
    vals, meta, bad = oracle.pack_two_four(Wh, M)
    assert bad == want_bad
    back = oracle.unpack_two_four(vals, meta, n)
    for row in range(m):
        for g in range(n // 4):
            sl = slice(4 * g, 4 * g + 4)
            if (~M[row, sl]).sum() <= 2:
                assert np.array_equal(back[row, sl], Wh[row, sl])


@pytest.mark.parametrize("nm", ["2:4", "4:8", "16:32", "16:64", "3:8"])
def test_nm_exact_groups(nm):
    W, _, _, _, _, U = _layer(12, 9, 64, 300)
    N, M = map(int, nm.split(":"))
    Wh, mask, _ = oracle.prune(W, U, nm, 64)
    g = mask.reshape(W.shape[0], -1, M).sum(axis=2)
    assert np.all(g == M - N)
    assert np.all(Wh[mask] == 0.0) and not np.any(np.signbit(Wh[mask]))


def test_nm_group_table_from_page():
    with open(os.path.join(GOLDEN, "nm_groups.json")) as f:
        fx = json.load(f)
    W, _, _, _, _, U = _layer(13, 4, 128, 400)
    for N, M, sparsity in fx["groups"]:
        _, mask, _ = oracle.prune(W, U, f"{N}:{M}", 128)
        assert mask.mean() == pytest.approx(sparsity, abs=0)


def test_compression_ratio_table_counts():
    with open(os.path.join(GOLDEN, "compression_ratios.json")) as f:
        fx = json.load(f)
    W, _, _, _, _, U = _layer(14, 30, 60, 300)
    m, n = W.shape
    for ratio, printed in fx["ratios"]:
        p = 1.0 - 1.0 / ratio
        assert p == pytest.approx(printed, abs=0.005)
        _, mask, _ = oracle.prune(W, U, p, n)
        assert mask.sum() == math.floor(p * m * n)


def test_sparsity_zero_and_one():
    W, _, _, _, _, U = _layer(15, 5, 33, 100)
    Wh, M, eps = oracle.prune(W, U, 0.0, 8)
    assert not M.any() and np.array_equal(Wh, W) and np.all(eps == 0)
    Wh, M, _ = oracle.prune(W, U, 1.0, 8)
    assert M.all() and np.all(Wh == 0.0) and not np.any(np.signbit(Wh))


def test_worked_two_four_example_identity_hessian():
    with open(os.path.join(GOLDEN, "two_four_example.json")) as f:
        fx = json.load(f)
    W = np.array([fx["dense"]])
    H = 7.0 * np.eye(4)
    Hd, _ = oracle.dampen(H, 0.01)
    U = oracle.inverse_upper_factor(Hd)
    Wh, mask, _ = oracle.prune(W, U, "2:4", 4)
    assert np.array_equal(Wh[0], np.array(fx["two_four"]))


def test_identity_hessian_is_magnitude_pruning():
    r = rng0(16)
    W = r.standard_normal((6, 40))
    Hd, _ = oracle.dampen(3.0 * np.eye(40), 0.01)
    U = oracle.inverse_upper_factor(Hd)
    Wh, M, _ = oracle.prune(W, U, 0.5, 20)
    for j in (0, 20):
        blk = np.abs(W[:, j:j + 20]).ravel()
        thr = np.sort(blk)[59]
        assert np.array_equal(M[:, j:j + 20].ravel(), blk <= thr)
    assert np.array_equal(Wh[~M], W[~M])


def test_diagonal_hessian_is_squared_wanda_score():
    # Diagonal H: no compensation, saliency w^2 (H_jj + lambda), i.e. the square
    # of the |w| * ||x_j|| score with the damped column norm.
    r = rng0(17)
    n = 32
    X = r.standard_normal((64, n)) * np.exp(r.standard_normal(n))[None, :]
    H = np.diag(np.sum(X * X, axis=0))
    Hd, lam = oracle.dampen(H, 0.01)
    U = oracle.inverse_upper_factor(Hd)
    W = r.standard_normal((8, n))
    Wh, M, _ = oracle.prune(W, U, "2:4", 32)
    score = np.abs(W) * np.sqrt(np.diag(H) + lam)[None, :]
    for g in range(0, n, 4):
        lowest = np.argsort(score[:, g:g + 4], axis=1)[:, :2]
        expect = np.zeros((8, 4), dtype=bool)
        np.put_along_axis(expect, lowest, True, axis=1)
        assert np.array_equal(M[:, g:g + 4], expect)
    assert np.array_equal(Wh[~M], W[~M])


def test_scale_invariance_bitwise():
    W, X, _, _, _, _ = _layer(18, 6, 24, 90)
    a = oracle.solve_layer(W, [X], 0.5, 8)
    b = oracle.solve_layer(W, [2.0 * X], 0.5, 8)
    assert np.array_equal(a["mask"], b["mask"])
    assert np.array_equal(a["W_hat"], b["W_hat"])


def test_row_permutation_equivariance_nm():
    W, _, _, _, _, U = _layer(19, 10, 32, 120)
    perm = rng0(3).permutation(10)
    Wa, Ma, _ = oracle.prune(W, U, "2:4", 16)
    Wb, Mb, _ = oracle.prune(W[perm], U, "2:4", 16)
    assert np.array_equal(Ma[perm], Mb) and np.array_equal(Wa[perm], Wb)


@pytest.mark.parametrize("pat", [0.5, "0.5/row", "2:4", "4:8"])
def test_free_set_route_matches_cholesky_route(pat):
    W, _, _, Hd, _, U = _layer(20, 7, 48, 200)
    a = oracle.prune(W, U, pat, 16)
    b = oracle.prune_free_set(W, Hd, pat, 16)
    assert np.array_equal(a[1], b[1])
    assert np.abs(a[0] - b[0]).max() < 1e-12
    assert np.allclose(a[2], b[2], rtol=1e-10)


def _lazy_blocked_reference(W, U, p, B):
    """Independent lazy batched formulation (the algebra the GPU path uses):
    sweep a block with updates confined to the block, then apply the block's
    errors to the trailing columns in one product."""
    Wh = W.astype(np.float64).copy()
    m, n = Wh.shape
    mask = np.zeros((m, n), dtype=bool)
    for i1 in range(0, n, B):
        i2 = min(n, i1 + B)
        w = i2 - i1
        blk = Wh[:, i1:i2].copy()
        s = blk ** 2 / np.diag(U)[i1:i2][None, :] ** 2
        k = math.floor(p * m * w)
        keys = sorted((s[r, c], r * n + i1 + c, r, c) for r in range(m) for c in range(w))
        bm = np.zeros((m, w), dtype=bool)
        for _, _, r, c in keys[:k]:
            bm[r, c] = True
        Err = np.zeros((m, w))
        for c in range(w):
            e = np.where(bm[:, c], blk[:, c] / U[i1 + c, i1 + c], 0.0)
            blk[:, c:] -= np.outer(e, U[i1 + c, i1:i2][c:])
            blk[bm[:, c], c] = 0.0
            Err[:, c] = e
        Wh[:, i1:i2] = blk
        mask[:, i1:i2] = bm
        Wh[:, i2:] -= Err @ U[i1:i2, i2:]
    return Wh, mask


def test_unbatched_equals_lazy_batched():
    W, _, _, _, _, U = _layer(21, 9, 45, 200)
    Wa, Ma, _ = oracle.prune(W, U, 0.5, 16)
    Wb, Mb = _lazy_blocked_reference(W, U, 0.5, 16)
    assert np.array_equal(Ma, Mb)
    assert np.abs(Wa - Wb).max() < 1e-13


# ----------------------------------------------------------------------------
# a8 reconstruction error
# ----------------------------------------------------------------------------

def test_reconstruction_error_paths_and_damping_identity():
    W, X, H, Hd, lam, U = _layer(22, 6, 30, 150)
    Wh, M, eps = oracle.prune(W, U, 0.5, 10)
    E = oracle.reconstruction_error(W, Wh, [X[:70], X[70:]])
    E_H = oracle.reconstruction_error_from_hessian(W, Wh, H)
    assert E == pytest.approx(E_H, rel=1e-11)
    # damped error = sum of e^2; undamped = damped - lambda ||W - Ŵ||^2
    assert E == pytest.approx(eps.sum() - lam * np.sum((W - Wh) ** 2), rel=1e-9)
    assert oracle.reconstruction_error(W, W, [X]) == 0.0
