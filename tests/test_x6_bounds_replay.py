"""Host replay of the address arithmetic of the split-product GEMM core's
two-buffer form (tile_gemm_x6_short in gemm_x6.h) where the library runs it:
the factorisation's next-column update (col_update_kernel, 64 x 64 quarters)
and the per-block lazy update (lazy_kernel<true, 64, true>); and of the
T = 128, four-chunk form inside the factor's fused panel launch, whose LDS
is the panel's.

Every global element offset each thread forms (operand loads, the C tile read
ahead, the epilogue's writes) is checked against the extent of the buffer it
points into, and every LDS offset against the workgroup's LDS, for the
launches the host code issues on the shapes the GPU tests and the benchmark
use.  The expressions mirror the device code line for line (loaders
RowsX6V / ColsX6T / CTileV, the launch loops of factor.hip and prune.hip);
nothing here runs on a GPU.
"""

import math

import numpy as np
import pytest

GBK, XS, NB, EGK, SB, NCU = 32, 32 + 8, 128, 512, 128, 256
TID = np.arange(256)


def cdiv(a, b):
    return -(-a // b)


def x6lds(T):
    plane = T * XS
    oper = 3 * plane
    nbytes = 2 * oper * 2
    epi = T * (T + 4) * 4
    return {"PLANE": plane, "OPER": oper, "SIZE": max(nbytes, epi), "SHORT": max(2 * nbytes, epi)}


def rows_x6v_load(T, full, ld, rows, kend, k0):
    """element offsets (relative to src) of RowsX6V<T, FULL>::load(k0)"""
    k4 = (TID & 7) * 4
    r0 = TID >> 3
    out = []
    for u in range(T // 32):
        if full or (rows == T and k0 + GBK <= kend and ld < (1 << 24)):
            base = 32 * u * ld + k0 + r0 * ld + k4
        else:
            k = k0 + k4
            kc = np.where(k < kend, k, kend - 4)
            r = r0 + 32 * u
            rc = np.where(r < rows, r, rows - 1)
            base = rc * ld + kc
        out.append(base[:, None] + np.arange(4)[None, :])
    return np.concatenate(out, axis=1)


def cols_x6t_load(T, full, ld, cols, kend, k0):
    """element offsets of ColsX6T<T, FULL>::load(k0)"""
    KT = GBK * T // 256
    j = TID % T
    kb = (TID // T) * KT
    out = []
    for u in range(KT):
        if full or (cols == T and k0 + GBK <= kend):
            off = (k0 + kb + u) * ld + j
        else:
            jc = np.where(j < cols, j, cols - 1)
            k = k0 + kb + u
            kc = np.where(k < kend, k, kend - 1)
            off = kc * ld + jc
        out.append(off)
    return np.stack(out, axis=1)


def ctile_rows(T, rows):
    """row / column offsets of CTileV<T>::load (reads, rows clamped) and of
    tile_sub_pre's writes (rows < rows)."""
    RPP = 256 // (T // 4)
    c4 = (TID % (T // 4)) * 4
    r0 = TID // (T // 4)
    rd, wr = [], []
    for rr in range(T // RPP):
        r = r0 + rr * RPP
        rc = np.where(r < rows, r, rows - 1)
        rd.append((rc, c4))
        wr.append((r[r < rows], c4[r < rows]))
    return rd, wr


def lds_short_max(T):
    """largest bf16 index tile_gemm_x6_short writes or reads (two buffers)"""
    L = x6lds(T)
    k4 = (TID & 7) * 4
    r0 = TID >> 3
    hi = 0
    for c in (0, 1):
        Pl = (c & 1) * 2 * L["OPER"]
        Ql = Pl + L["OPER"]
        for base in (Pl, Ql):
            # RowsX6V store: 3 planes, rows r0 + 32u, k4 .. k4 + 3
            for u in range(T // 32):
                hi = max(hi, int(np.max(base + 2 * L["PLANE"] + (r0 + 32 * u) * XS + k4 + 3)))
        # ColsX6T store: row j, k offsets kb + 4q .. + 3
        KT = GBK * T // 256
        j = TID % T
        kb = (TID // T) * KT
        hi = max(hi, int(np.max(Ql + 2 * L["PLANE"] + j * XS + kb + KT - 1)))
        # tile_mma_x6 reads: rows prow/qrow + 16 i, k .. k + 7
        lane = TID & 63
        prow = ((TID >> 6) >> 1) * (T // 2) + (lane & 15)
        k = (lane >> 4) * 8
        for i in range(T // 32):
            hi = max(hi, int(np.max(Ql + 2 * L["PLANE"] + (prow + 16 * i) * XS + k + 7)))
    return hi


def test_lds_extents():
    # two-buffer T = 64: the static array of col_update_kernel / lazy_kernel
    L64 = x6lds(64)
    assert 2 * (lds_short_max(64) + 1) <= L64["SHORT"]
    assert 64 * 68 * 4 <= L64["SHORT"]  # the epilogue staging tile
    # T = 128, four chunks, inside the fused panel launch: the panel's LDS
    panel_lds = 2 * NB * 132 * 4 + 4
    assert 2 * (lds_short_max(128) + 1) <= panel_lds
    assert 128 * 132 * 4 <= panel_lds


def check_in(offs, extent, what):
    offs = np.asarray(offs)
    if offs.size == 0:
        return
    assert offs.min() >= 0 and offs.max() < extent, (what, int(offs.min()), int(offs.max()), extent)


@pytest.mark.parametrize("kw", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [200, 1000, 4096, 4224, 11008, 28672])
def test_col_update_offsets(n, kw):
    """col_update_kernel<KW> for every panel step k: block column kl + 1 of the
    update of panels k .. kl = k + kw - 1 (kw > 1 groups panels, K = 128 kw,
    streamed by the pipelined core; kw = 1 is the two-buffer core, K = 128):
    the C quarter and the P and Q loaders (RowsX6V<64, true>) against the
    n_pad x n_pad A and Y matrices."""
    n_pad = cdiv(n, NB) * NB
    nblk = n_pad // NB
    ext = n_pad * n_pad
    ks = [k for k in range(nblk) if k + kw < nblk]
    if nblk > 40:
        ks = ks[:3] + ks[-4:]
    for k in ks:
        kl = k + kw - 1
        t = nblk - kl - 1
        tiles = t + kl + 1
        # the first and last tiles of each kind (every other tile's offsets
        # lie between theirs)
        idxs = sorted({0, 1, t - 1, t, t + 1, tiles - 2, tiles - 1} & set(range(tiles)))
        for bid in [4 * i + q for i in idxs for q in range(4)]:
            idx, qr, qc = bid >> 2, (bid >> 1) & 1, bid & 1
            if idx < t:
                if idx == 0 and qr < qc:
                    continue
                lb, mb = kl + 1 + idx, kl + 1
                C = lb * NB * n_pad + mb * NB          # into A
                P = lb * NB * n_pad + k * NB           # into A
                Q = mb * NB * n_pad + k * NB           # into A
            else:
                c, lb = idx - t, kl + 1
                C = c * NB * n_pad + lb * NB           # into Y
                P = c * NB * n_pad + k * NB            # into Y
                Q = lb * NB * n_pad + k * NB           # into A
            # the K = kw * 128 columns read stay in the row (block columns k
            # .. k + kw - 1)
            assert (P % n_pad) + kw * NB <= n_pad and (Q % n_pad) + kw * NB <= n_pad
            Cq = C + qr * 64 * n_pad + qc * 64
            rd, wr = ctile_rows(64, 64)
            for (r, c4) in rd + wr:
                check_in(Cq + r[:, None] * n_pad + c4[:, None] + np.arange(4), ext, ("C", n, k, bid))
            for c in range(kw * NB // GBK):
                check_in(P + qr * 64 * n_pad + rows_x6v_load(64, True, n_pad, 64, kw * NB, c * GBK), ext,
                         ("P", n, k, bid, c))
                check_in(Q + qc * 64 * n_pad + rows_x6v_load(64, True, n_pad, 64, kw * NB, c * GBK), ext,
                         ("Q", n, k, bid, c))


@pytest.mark.parametrize("kw", [2, 3, 4])
@pytest.mark.parametrize("n", [4224, 11008, 28672])
def test_grouped_rest_update_tiles(n, kw):
    """update_body<KW> (UPD_REST) tile map: every SYRK tile lies in A's lower
    block triangle beyond block column k + kw, every inverse tile in Y's upper
    block triangle, each tile once."""
    n_pad = cdiv(n, NB) * NB
    nblk = n_pad // NB
    for k in [0, 1, nblk // 2, nblk - 6, nblk - 1 - kw]:
        if k < 0 or k + kw >= nblk:
            continue
        kl = k + kw - 1
        s0 = kl + 2
        ts = nblk - s0
        nsyrk = ts * (ts + 1) // 2
        t = nblk - kl - 1
        total = (t - 1) * t // 2 + (kl + 1) * (t - 1)
        assert total == nsyrk + (kl + 1) * ts
        seen = set()
        for idx in range(total):
            if idx < nsyrk:
                l = (math.isqrt(8 * idx + 1) - 1) // 2
                m = idx - l * (l + 1) // 2
                lb, mb = s0 + l, s0 + m
                assert s0 <= mb <= lb < nblk
                seen.add(("A", lb, mb))
            else:
                j = idx - nsyrk
                c, lb = j % (kl + 1), s0 + j // (kl + 1)
                assert c <= kl < lb < nblk
                seen.add(("Y", c, lb))
        assert len(seen) == total  # each tile once


def lazy_launches(m, n, B):
    """(E offset, K, c_begin, c_end, k0) of every lazy update the prune loop
    issues for one matrix of m rows."""
    GK = (EGK // B) * B
    out = []
    for i1 in range(0, n, B):
        w = min(B, n - i1)
        g0 = (i1 // GK) * GK
        g_end = min(n, g0 + GK)
        i2 = i1 + w
        if i2 < g_end:
            out.append((i1 - g0, w, i2, g_end, i1))
        elif g_end < n:
            out.append((0, g_end - g0, g_end, n, g0))
    return out


@pytest.mark.parametrize("m,n,B", [(64, 128, 32), (256, 512, 128), (384, 512, 128), (200, 1000, 128),
                                   (130, 384, 64), (96, 256, 32), (4096, 4096, 128), (11008, 4096, 128),
                                   (4096, 11008, 128), (8192, 28672, 128)])
def test_lazy_short_offsets(m, n, B):
    """lazy_kernel<true, 64, true> (the launches where the 64 x 64 tile and
    the two-buffer core are chosen): the W tile read ahead and written back,
    the error rows (RowsX6V<64>, row stride EGK) and the U rows
    (ColsX6T<64>) against W (m x n), Err (m x EGK) and U (n x n)."""
    seen = 0
    launches = lazy_launches(m, n, B)
    if m * n > (1 << 24):  # large layers: the first and the last launches of the sweep
        launches = launches[:6] + launches[-6:]
    for (eoff, K, cb, ce, k0) in launches:
        t128 = cdiv(ce - cb, 128) * cdiv(m, 128)
        vec = (eoff % 4 == 0) and (K % 4 == 0)
        if t128 >= 2 * NCU or not (vec and K <= SB):
            continue
        seen += 1
        gx, gy = cdiv(ce - cb, 64), cdiv(m, 64)
        xs = range(gx) if gx * gy <= 4096 else sorted({0, 1, gx - 2, gx - 1} & set(range(gx)))
        ys = range(gy) if gx * gy <= 4096 else sorted({0, 1, gy - 2, gy - 1} & set(range(gy)))
        for bx in xs:
            for by in ys:
                r0, c0 = by * 64, cb + bx * 64
                rows, cols = min(64, m - r0), min(64, ce - c0)
                C = r0 * n + c0
                cpre = cols == 64 and n % 4 == 0 and C % 4 == 0
                rd, wr = ctile_rows(64, rows)
                if cpre:
                    for (r, c4) in rd + wr:
                        check_in(C + r[:, None] * n + c4[:, None] + np.arange(4), m * n, ("W", m, n, c0, r0))
                for c in range(cdiv(K, GBK)):
                    e = eoff + r0 * EGK + rows_x6v_load(64, False, EGK, rows, K, c * GBK)
                    check_in(e, m * EGK, ("E", m, n, c0, r0, c))
                    col = (e - eoff) % EGK  # the error columns stay inside the row's group
                    assert col.max() + eoff < EGK
                    u = k0 * n + c0 + cols_x6t_load(64, False, n, cols, K, c * GBK)
                    check_in(u, n * n, ("U", m, n, c0, r0, c))
                if not cpre:
                    # tile_sub_from, element path: rows < rows, columns < cols
                    RPP = 16
                    c4 = (TID % 16) * 4
                    rr0 = TID // 16
                    for rr in range(64 // RPP):
                        r = rr0 + rr * RPP
                        ok = r < rows
                        for e4 in range(4):
                            okc = ok & (c4 + e4 < cols)
                            check_in((C + r * n + c4 + e4)[okc], m * n, ("W-", m, n))
    assert seen > 0 or m * n >= 4096 * 4096


def test_x6_short_chunk_count():
    # the two-buffer core holds NCH = SB / GBK register sets; every K it is
    # given (a block width <= SB, or the 128-wide panel) fits
    for K in range(1, SB + 1):
        assert math.ceil(K / GBK) <= SB // GBK
