"""Planted mistakes in copies of the oracle (CPU only) must each fail a pin.

Each mutant wraps the real oracle and breaks one step the way a plausible bug
would: a floor instead of a ceiling, a missing square root, the wrong end of
the ranking, the wrong tie order, an unsorted index list, a dropped term, a
wrong sign, a transposed operand, a lost scale factor.  If a mutant passed
every pin, the pins could not tell that bug from the method.
"""
import math
import types

import numpy as np
import pytest

import pins


def _mutant(oracle, **over):
    ns = types.SimpleNamespace(k_of=oracle.k_of, colnorm=oracle.colnorm, topk=oracle.topk,
                               reduced_product=oracle.reduced_product)
    for k, v in over.items():
        setattr(ns, k, v(oracle))
    return ns


def _stable_desc(s, k):
    return np.sort(np.argsort(-np.asarray(s), kind="stable")[:k]).astype(np.int32)


MUTANTS = {
    "k_floor": dict(k_of=lambda o: (lambda r, d: max(1, int(r * d)) if 0 < r <= 1 and d > 0 else 0)),
    "k_plain_ceil": dict(k_of=lambda o: (lambda r, d: math.ceil(r * d) if 0 < r <= 1 and d > 0 else 0)),
    "norm_no_sqrt": dict(colnorm=lambda o: (lambda A: o.colnorm(A) ** 2)),
    "norm_l1": dict(colnorm=lambda o: (lambda A: np.abs(np.asarray(A, np.float64)).sum(0))),
    "norm_rows": dict(colnorm=lambda o: (lambda A: o.colnorm(np.asarray(A, np.float64).T)[: np.shape(A)[1]]
                                         if np.shape(A)[0] >= np.shape(A)[1] else np.linalg.norm(A, axis=0) * 1.5)),
    "topk_smallest": dict(topk=lambda o: (lambda s, k: _stable_desc(-np.asarray(s), k))),
    "topk_ties_high": dict(topk=lambda o: (lambda s, k: np.sort(
        (len(s) - 1 - np.argsort(-np.asarray(s)[::-1], kind="stable"))[:k]).astype(np.int32))),
    "topk_score_order": dict(topk=lambda o: (lambda s, k: np.argsort(-np.asarray(s), kind="stable")[:k]
                                             .astype(np.int32))),
    "topk_off_by_one": dict(topk=lambda o: (lambda s, k: o.topk(s, max(1, k - 1)) if k > 1 else o.topk(s, k))),
    "product_drop_last": dict(reduced_product=lambda o: (lambda A, B, idx, alpha=1.0, rows=None, threads=None:
                                                         o.reduced_product(A, B, idx[:-1], alpha, rows, threads))),
    "product_sign": dict(reduced_product=lambda o: (lambda A, B, idx, alpha=1.0, rows=None, threads=None:
                                                    -o.reduced_product(A, B, idx, alpha, rows, threads))),
    "product_transposed_B": dict(reduced_product=lambda o: (
        lambda A, B, idx, alpha=1.0, rows=None, threads=None:
        o.reduced_product(A, np.ascontiguousarray(np.asarray(B).T) if np.shape(B)[0] == np.shape(B)[1]
                          else np.asarray(B)[::-1], idx, alpha, rows, threads))),
    "product_no_alpha": dict(reduced_product=lambda o: (lambda A, B, idx, alpha=1.0, rows=None, threads=None:
                                                        o.reduced_product(A, B, idx, 1.0, rows, threads))),
    "product_shifted_index": dict(reduced_product=lambda o: (
        lambda A, B, idx, alpha=1.0, rows=None, threads=None:
        o.reduced_product(A, B, np.minimum(np.asarray(idx) + 1, np.shape(A)[1] - 1).astype(np.int32),
                          alpha, rows, threads))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, oracle_mod):
    impl = _mutant(oracle_mod, **MUTANTS[name])
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
