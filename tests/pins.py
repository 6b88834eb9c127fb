"""Pins for the CPU oracle: checks against what the paper and mathematics fix.

Each ``pin_*`` function takes an implementation object with the oracle's
interface (``k_of``, ``colnorm``, ``topk``, ``reduced_product``) and raises
AssertionError when it disagrees with an independent source of truth:

* closed forms and hand-worked numbers (``tests/golden/hand_rmm_2x6.json``);
* library routines that compute the same definition another way
  (``numpy.linalg.norm``, ``numpy.argsort(kind="stable")``, ``numpy @``);
* exact rational arithmetic (``fractions.Fraction``) for ceil(rho d);
* brute force over every index subset of tiny problems (Theorem 1, App. E.1);
* identities and inequalities of App. E (eqs. 9, 12, 13, 14, 17, 18) and the
  tight construction of Remark 1.

``test_oracle_pins.py`` runs every pin on the real oracle; ``test_oracle_
mutants.py`` runs them on copies of the oracle with planted mistakes and
requires each mistake to be caught, which shows the pins have teeth.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_rmm_2x6.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


# ----------------------------------------------------------------------------- k = ceil(rho d)

K_TABLE = [
    # (rho, d, k): |I| = ceil(rho d) (Sec. 3.2) for the workloads' sizes and edge cases
    (0.5, 4096, 2048), (0.7, 4096, 2868), (0.8, 4096, 3277), (1.0, 4096, 4096),
    (0.5, 14336, 7168), (0.7, 14336, 10036), (0.8, 14336, 11469), (1.0, 14336, 14336),
    (0.8, 8192, 6554), (0.5, 128, 64), (0.5, 256, 128),
    (0.07, 100, 7),    # 0.07*100 evaluates to 7.000000000000001 in binary
    (0.3, 10, 3),      # 0.3*10 evaluates to 3.0000000000000004
    (0.7, 10, 7), (0.1, 3, 1), (1e-9, 10, 1), (1.0, 1, 1), (0.5, 1, 1), (0.99, 1000, 990),
]
K_INVALID = [(0.0, 10), (-0.5, 10), (1.0000001, 10), (float("nan"), 10), (0.5, 0), (0.5, -3)]


def pin_k_table(impl):
    for rho, d, k in K_TABLE:
        got = impl.k_of(rho, d)
        assert got == k, f"k_of({rho}, {d}) = {got}, expected {k}"
    for rho, d in K_INVALID:
        assert impl.k_of(rho, d) == 0, f"k_of({rho}, {d}) should be invalid (0)"


def pin_k_exact_fraction(impl, trials=3000, seed=11):
    """ceil of the exact rational rho*d, with rho read as the decimal it was written as."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        digits = int(rng.integers(1, 5))
        num = int(rng.integers(1, 10 ** digits + 1))
        text = f"{num / 10 ** digits:.{digits}f}"
        rho = float(text)
        if rho > 1.0:
            continue
        d = int(rng.integers(1, 50000))
        exact = math.ceil(Fraction(text) * d)
        got = impl.k_of(rho, d)
        assert got == exact, f"k_of({text}, {d}) = {got}, exact ceil = {exact}"


# ----------------------------------------------------------------------------- column norms

def pin_colnorm_golden(impl):
    g = golden()
    s = impl.colnorm(np.array(g["A"], dtype=np.float64))
    assert np.array_equal(s, np.array(g["colnorms"]["values"], dtype=np.float64)), s


def pin_colnorm_library(impl, seed=12):
    rng = np.random.default_rng(seed)
    for n, d in [(1, 7), (5, 3), (64, 256), (300, 17), (2, 1)]:
        A = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
        ref = np.linalg.norm(A, axis=0)
        got = impl.colnorm(A)
        assert got.shape == (d,)
        assert np.max(np.abs(got - ref) / ref) < 1e-13, (n, d)


def pin_colnorm_single_row(impl, seed=13):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((1, 33))
    assert np.array_equal(impl.colnorm(a), np.abs(a[0])), "n = 1 must give |a_j| exactly"


def pin_colnorm_pow2_scaling(impl, seed=14):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((9, 12))
    s = impl.colnorm(A)
    for p in (-7, 3, 11):
        assert np.array_equal(impl.colnorm(A * 2.0 ** p), s * 2.0 ** p)


# ----------------------------------------------------------------------------- TopK selection

def pin_topk_golden(impl):
    g = golden()
    s = np.array(g["colnorms"]["values"], dtype=np.float64)
    for sel in g["selections"]:
        k = impl.k_of(sel["rho"], s.size)
        assert k == sel["k"], (sel, k)
        idx = impl.topk(s, k)
        assert list(idx) == sel["idx"], (sel, list(idx))


def pin_topk_library(impl, seed=15):
    """Same result as numpy's stable argsort of -s (stable = ties keep index order)."""
    rng = np.random.default_rng(seed)
    for d in (1, 2, 7, 64, 1000, 4099):
        s = np.abs(rng.standard_normal(d))
        s[rng.integers(0, d, size=d // 3)] = s[0]  # plenty of exact ties
        for k in sorted({1, d // 3 or 1, d // 2 or 1, d}):
            ref = np.sort(np.argsort(-s, kind="stable")[:k])
            got = impl.topk(s, k)
            assert got.dtype == np.int32
            assert np.array_equal(got, ref), (d, k)


def pin_topk_ties(impl):
    # duplicate and zero columns: the lower index wins every tie
    A = np.array([[1.0, 2.0, 1.0, 0.0, 2.0, 0.0],
                  [1.0, 0.0, 1.0, 0.0, 0.0, 0.0]])
    s = impl.colnorm(A)      # [sqrt2, 2, sqrt2, 0, 2, 0]
    assert list(impl.topk(s, 1)) == [1]
    assert list(impl.topk(s, 2)) == [1, 4]
    assert list(impl.topk(s, 3)) == [0, 1, 4]
    assert list(impl.topk(s, 5)) == [0, 1, 2, 3, 4]
    z = np.zeros(5)
    assert list(impl.topk(z, 2)) == [0, 1]


def pin_topk_bruteforce(impl, seed=16):
    """Theorem 1 (App. E.1): the selected set minimises the worst case of the
    Prop. 1 surrogate over unknown row energies b >= 0, sum b^2 <= 1.

    The inner maximum is computed here as the l2 norm of the dropped scores
    (eq. 9, the l2 ball is self-dual on the nonnegative orthant); it is first
    checked against random feasible b and against Remark 1's adversary.
    """
    rng = np.random.default_rng(seed)
    for d in range(1, 10):
        for trial in range(3):
            n = int(rng.integers(1, 5))
            A = rng.standard_normal((n, d))
            if trial == 2 and d > 2:
                A[:, 1] = A[:, 0]  # an exact tie
            alpha = np.linalg.norm(A, axis=0)
            s = impl.colnorm(A)
            for k in range(1, d + 1):
                best, minimisers = None, []
                for I in itertools.combinations(range(d), k):
                    drop = np.setdiff1d(np.arange(d), I)
                    val = float(np.sum(alpha[drop] ** 2))
                    if best is None or val < best - 1e-12 * max(best, 1e-300):
                        best, minimisers = val, [I]
                    elif abs(val - best) <= 1e-12 * max(best, 1e-300):
                        minimisers.append(I)
                got = tuple(int(x) for x in impl.topk(s, k))
                assert got in minimisers, (d, k, got, minimisers[:3])
                if k < d:  # inner maximum of eq. (8) for the chosen set
                    drop = np.setdiff1d(np.arange(d), got)
                    closed = math.sqrt(float(np.sum(alpha[drop] ** 2)))
                    b = np.abs(rng.standard_normal((200, d)))
                    b /= np.linalg.norm(b, axis=1, keepdims=True)
                    assert np.all(b[:, drop] @ alpha[drop] <= closed * (1 + 1e-12))
                    if closed > 0:
                        adv = np.zeros(d)
                        adv[drop] = alpha[drop] / closed  # Remark 1
                        assert abs(adv @ alpha - closed) <= 1e-12 * closed


def pin_topk_nesting(impl, seed=17):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((20, 97))
    s = impl.colnorm(A)
    prev = set()
    for rho in (0.1, 0.3, 0.5, 0.7, 0.8, 0.9, 1.0):
        cur = set(impl.topk(s, impl.k_of(rho, 97)).tolist())
        assert prev <= cur
        prev = cur


def pin_topk_permutation(impl, seed=18):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((6, 40)) * np.exp(rng.standard_normal(40))
    B = rng.standard_normal((40, 5))
    pi = rng.permutation(40)
    k = impl.k_of(0.6, 40)
    I = impl.topk(impl.colnorm(A), k)
    Ip = impl.topk(impl.colnorm(A[:, pi]), k)
    inv = np.argsort(pi)
    assert np.array_equal(np.sort(pi[Ip]), I)           # same columns, relabelled
    assert np.array_equal(np.sort(inv[I]), Ip)
    Y = impl.reduced_product(A, B, I)
    Yp = impl.reduced_product(A[:, pi], B[pi, :], Ip)
    assert _rel(Yp, Y) < 1e-13


# ----------------------------------------------------------------------------- reduced product

def pin_product_golden(impl):
    g = golden()
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    s = impl.colnorm(A)
    for p in g["products"]:
        idx = impl.topk(s, impl.k_of(p["rho"], A.shape[1]))
        Y = impl.reduced_product(A, B, idx, p["alpha"])
        assert np.array_equal(Y, np.array(p["Y"], dtype=np.float64)), (p, Y)
    idx = impl.topk(s, impl.k_of(0.5, 6))
    E = A @ B - impl.reduced_product(A, B, idx)
    assert np.array_equal(E, np.array(g["rho05_error"]["AB_minus_Y"], dtype=np.float64))


def pin_product_dense(impl, seed=19):
    """rho = 1 keeps every index, so the result is the full product (Sec. 3.2)."""
    rng = np.random.default_rng(seed)
    for n, d, m in [(1, 1, 1), (3, 5, 7), (17, 33, 9), (64, 256, 128)]:
        A = rng.standard_normal((n, d))
        B = rng.standard_normal((d, m))
        idx = impl.topk(impl.colnorm(A), impl.k_of(1.0, d))
        assert np.array_equal(idx, np.arange(d, dtype=np.int32))
        Y = impl.reduced_product(A, B, idx)
        assert Y.shape == (n, m)
        assert _rel(Y, A @ B) < 1e-13, (n, d, m)


def pin_product_complement(impl, seed=20):
    """eq. (13): AB - A[:,I]B[I,:] equals the product over the dropped indices."""
    rng = np.random.default_rng(seed)
    for n, d, m, rho in [(8, 30, 11, 0.5), (31, 64, 5, 0.8), (2, 9, 40, 0.3)]:
        A = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
        B = rng.standard_normal((d, m))
        idx = impl.topk(impl.colnorm(A), impl.k_of(rho, d))
        drop = np.setdiff1d(np.arange(d), idx)
        E = A @ B - impl.reduced_product(A, B, idx)
        assert _rel(E, A[:, drop] @ B[drop, :]) < 1e-12


def pin_product_bounds(impl, seed=21):
    """eqs. (12), (14), (17) hold and eq. (18): no other set leaves less A-energy."""
    rng = np.random.default_rng(seed)
    for n, d, m, rho in [(16, 50, 12, 0.5), (5, 20, 30, 0.7), (40, 64, 8, 0.9)]:
        A = rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))
        B = rng.standard_normal((d, m)) * np.exp(rng.standard_normal(d))[:, None]
        k = impl.k_of(rho, d)
        idx = impl.topk(impl.colnorm(A), k)
        drop = np.setdiff1d(np.arange(d), idx)
        err = np.linalg.norm(A @ B - impl.reduced_product(A, B, idx))
        a = np.linalg.norm(A, axis=0)
        b = np.linalg.norm(B, axis=1)
        prop1 = float(np.sum(a[drop] * b[drop]))
        cor1 = math.sqrt(np.sum(a[drop] ** 2)) * math.sqrt(np.sum(b[drop] ** 2))
        assert err <= prop1 * (1 + 1e-12) and prop1 <= cor1 * (1 + 1e-12)
        rel = err / (np.linalg.norm(A) * np.linalg.norm(B))
        eps_a = np.sum(a[drop] ** 2) / np.sum(a ** 2)
        eps_b = np.sum(b[drop] ** 2) / np.sum(b ** 2)
        assert rel <= math.sqrt(eps_a * eps_b) * (1 + 1e-12)
        assert float(np.sum(a[idx] ** 2) / np.sum(a ** 2)) >= k / d - 1e-12  # retained energy >= k/d
        resid = float(np.sum(a[drop] ** 2))
        for _ in range(50):
            other = rng.choice(d, size=k, replace=False)
            odrop = np.setdiff1d(np.arange(d), other)
            assert resid <= float(np.sum(a[odrop] ** 2)) * (1 + 1e-12)


def pin_product_tight(impl, seed=22):
    """Remark 1 / eq. (12) with equality: when every dropped column of A is a
    nonnegative multiple of one vector u and every dropped row of B a
    nonnegative multiple of one vector v, the dropped terms are all parallel
    and the triangle inequality is tight."""
    rng = np.random.default_rng(seed)
    n, d, m = 7, 12, 9
    u, v = rng.standard_normal(n), rng.standard_normal(m)
    A = rng.standard_normal((n, d)) * 10.0
    B = rng.standard_normal((d, m))
    ks = impl.k_of(0.5, d)
    idx = impl.topk(impl.colnorm(A), ks)
    drop = np.setdiff1d(np.arange(d), idx)
    A[:, drop] = np.outer(u, rng.uniform(0.1, 0.5, drop.size))  # small, parallel, still dropped
    B[drop, :] = np.outer(rng.uniform(0.5, 2.0, drop.size), v)
    idx = impl.topk(impl.colnorm(A), ks)
    assert np.array_equal(np.setdiff1d(np.arange(d), idx), drop)
    err = np.linalg.norm(A @ B - impl.reduced_product(A, B, idx))
    bound = float(np.sum(np.linalg.norm(A[:, drop], axis=0) * np.linalg.norm(B[drop, :], axis=1)))
    assert abs(err - bound) <= 1e-12 * bound


def pin_product_python_loops(impl, seed=23):
    """Pure-Python triple loop on a tiny case, exact-integer data (no rounding)."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-9, 10, size=(4, 7)).astype(np.float64)
    B = rng.integers(-9, 10, size=(7, 5)).astype(np.float64)
    idx = [0, 2, 3, 6]
    Y = impl.reduced_product(A, B, np.array(idx, dtype=np.int32), 3.0)
    for i in range(4):
        for c in range(5):
            acc = 0
            for j in idx:
                acc += int(A[i, j]) * int(B[j, c])
            assert Y[i, c] == 3 * acc


def pin_product_rows(impl, seed=24):
    """Sampled rows equal the matching rows of the full result, bit for bit."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((33, 20))
    B = rng.standard_normal((20, 6))
    idx = impl.topk(impl.colnorm(A), 11)
    full = impl.reduced_product(A, B, idx, 0.25)
    rows = [32, 0, 7, 7, 19]
    part = impl.reduced_product(A, B, idx, 0.25, rows=rows)
    assert np.array_equal(part, full[rows])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
