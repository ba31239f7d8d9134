"""The conv2d backward's gather, written out in Python, against the oracle.

The HIP backward takes x in quads (rows 2m, 2m+1 x columns 2n, 2n+1) and
gathers each dx element from the dy elements and taps that reach it, per
axis from a table chosen by the padding before that axis; db adds each dy
element once, the last column apart when two zeros pad the columns.  This
test restates those tables and that grid on the CPU, in float64, and checks
that they reproduce the oracle's scatter-form dx, dw and db for every
padding combination the kernels accept, on shapes with odd and even sizes,
empty axes and masked items.  It does not run the HIP code (the GPU parity
tests do); it pins the derivation the kernel is built on.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def terms(P, e):
    """(output offset, tap) pairs that reach input 2n + e along an axis with
    P + 1 zeros before it."""
    if P == 0:
        return [(0, 1)] if e == 0 else [(0, 2), (1, 0)]
    return [(0, 2), (1, 0)] if e == 0 else [(1, 1)]


def gather_bwd(x, w, L, dy, pads):
    B, T, F, C = x.shape
    pt0, pt1, pf0, pf1 = pads
    To, Fo = dy.shape[1], dy.shape[2]
    PR, PC = pt0 - 1, pf0 - 1
    NQt = max((T + 1) // 2, To)
    NQf = max((F + 1) // 2, Fo) if PC == 0 else max((F + 1) // 2, Fo - 1, 1 if Fo > 0 else 0)
    dx, dw, db = np.zeros_like(x), np.zeros((3, 3, C)), np.zeros(C)
    for b in range(B):
        ln = min(max(int(L[b]), 0), T)
        leno = 0 if ln <= 0 else min(max((ln + pt0 + pt1 - 3) // 2 + 1, 0), To)

        def g(r, c):
            return dy[b, r, c] if 0 <= r < leno and 0 <= c < Fo else np.zeros(C)

        def xv(r, c):
            return x[b, r, c] if r < ln and c < F else np.zeros(C)

        for m in range(NQt):
            for n in range(NQf):
                for er, ec in itertools.product(range(2), range(2)):
                    d = np.zeros(C)
                    for (oi, ti), (oj, tj) in itertools.product(terms(PR, er), terms(PC, ec)):
                        gv = g(m + oi, n + oj)
                        d += gv * w[ti, tj]
                        dw[ti, tj] += gv * xv(2 * m + er, 2 * n + ec)
                    r, c = 2 * m + er, 2 * n + ec
                    if r < T and c < F:
                        dx[b, r, c] = d if r < ln else 0.0
                db += g(m, n)
                if PC == 1 and n == NQf - 1:
                    db += g(m, n + 1)
    return dx, dw, db


PADS = list(itertools.product([1, 2], [0, 1, 2], [1, 2], [0, 1, 2]))


@pytest.mark.parametrize("T,F", [(7, 6), (8, 9), (1, 1), (2, 5), (0, 4), (5, 0), (9, 10)])
def test_gather_tables_reproduce_the_scatter_backward(T, F):
    rng = np.random.default_rng(T * 31 + F)
    B, C = 2, 3
    for pads in PADS:
        To = max(oracle.conv_out_len(T, 3, 2, pads[0], pads[1]), 0)
        Fo = max(oracle.conv_out_len(F, 3, 2, pads[2], pads[3]), 0)
        x = torch.as_tensor(rng.standard_normal((B, T, F, C)), dtype=torch.float32)
        w = torch.as_tensor(rng.standard_normal((3, 3, C)), dtype=torch.float32)
        dy = torch.as_tensor(rng.standard_normal((B, To, Fo, C)), dtype=torch.float32)
        L = [T, max(T - 3, 0)]
        rdx, rdw, rdb = oracle.dwconv2d_bwd(x, w, torch.tensor(L, dtype=torch.int32), dy, pads=pads)
        gdx, gdw, gdb = gather_bwd(x.double().numpy(), w.double().numpy(), L, dy.double().numpy(), pads)
        for name, a, r in (("dx", gdx, rdx), ("dw", gdw, rdw), ("db", gdb, rdb)):
            assert np.allclose(a, r, rtol=0, atol=1e-9), f"{name} differs at pads {pads}"


def test_a_dropped_term_is_caught():
    """The comparison can fail: without the last-column db term the causal
    columns lose dy's last column."""
    rng = np.random.default_rng(5)
    T, F, C, pads = 6, 8, 2, (2, 1, 2, 1)
    To, Fo = oracle.conv_out_len(T, 3, 2, 2, 1), oracle.conv_out_len(F, 3, 2, 2, 1)
    x = rng.standard_normal((1, T, F, C))
    w = rng.standard_normal((3, 3, C))
    dy = rng.standard_normal((1, To, Fo, C))
    _, _, db = gather_bwd(x, w, [T], dy, pads)
    assert np.allclose(db, dy.sum(axis=(0, 1, 2)))
    assert not np.allclose(db - dy[0, :, Fo - 1].sum(axis=0), dy.sum(axis=(0, 1, 2)))
