"""Oracle pieces beyond the four core functions: the GQA attention mapping,
the end-to-end ``rmm`` wrapper, diagnostics, determinism and the input gap
fix-up."""
import math

import numpy as np

import synthetic


def test_attention_gqa_mapping(oracle_mod):
    """Sec. 3.3: select on Q_h's column norms, take the same dimensions of the
    shared K head g = h // (H_q / H_kv), scale by 1/sqrt(d_h) (full d_h)."""
    rng = np.random.default_rng(30)
    hq, hkv, L, dh = 6, 2, 9, 8
    Q = rng.standard_normal((hq, L, dh)) * np.exp(rng.standard_normal((hq, 1, dh)))
    K = rng.standard_normal((hkv, L, dh))
    alpha = 1.0 / math.sqrt(dh)
    res = oracle_mod.attention_scores(Q, K, 0.5, alpha)
    for h, r in enumerate(res):
        g = h // (hq // hkv)
        I = np.sort(np.argsort(-np.linalg.norm(Q[h], axis=0), kind="stable")[:4])
        assert np.array_equal(r.idx, I)
        ref = alpha * (Q[h][:, I] @ K[g][:, I].T)
        assert np.max(np.abs(r.Y - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_rmm_wrapper_and_diagnostics(oracle_mod):
    g = __import__("pins").golden()
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    r = oracle_mod.rmm(A, B, 0.5)
    assert r.k == 3 and list(r.idx) == [0, 2, 3]
    assert np.array_equal(r.Y, np.array([[8, 12], [16, 16]], dtype=np.float64))
    dg = oracle_mod.diagnostics(A, B, r.idx)
    assert abs(dg["retained_energy"] - 294 / 324) < 1e-15
    assert abs(dg["prop1"] - (math.sqrt(10) + 12 * math.sqrt(2))) < 1e-13
    assert abs(dg["cor1"] - math.sqrt(30) * math.sqrt(20)) < 1e-12  # ||A_drop||_F^2 = 1+25+4, ||B_drop||_F^2 = 10+8+2
    # eq. (17): eps_A, eps_B and the relative bound, worked by hand in the golden file
    assert abs(dg["eps_A"] - 5 / 54) < 1e-15
    assert abs(dg["eps_B"] - 20 / 27) < 1e-15
    assert abs(dg["rel17"] - 10 / (27 * math.sqrt(2))) < 1e-15
    assert abs(dg["normA_F"] - 18) < 1e-13 and abs(dg["normB_F"] - math.sqrt(27)) < 1e-13
    rel_err = math.sqrt(g["rho05_error"]["frobenius_squared"]) / (dg["normA_F"] * dg["normB_F"])
    assert rel_err <= dg["rel17"]


def test_repeatable_and_thread_count_independent(oracle_mod):
    case = synthetic.make_case("c1")
    a = oracle_mod.rmm(case.A, case.B, 0.5, threads=1)
    b = oracle_mod.rmm(case.A, case.B, 0.5, threads=7)
    c = oracle_mod.rmm(case.A, case.B, 0.5)
    assert np.array_equal(a.idx, b.idx) and np.array_equal(a.idx, c.idx)
    assert np.array_equal(a.Y, b.Y) and np.array_equal(a.Y, c.Y)
    assert np.array_equal(a.s, b.s)


def test_gap_fixup_opens_every_boundary(oracle_mod):
    from oracle.fixup import enforce_gap
    case = synthetic.make_case("c2", scale=dict(n=64, d=512, m=64))
    ks = [oracle_mod.k_of(r, 512) for r in case.rhos]
    A, touched = enforce_gap(case.A, ks, "bf16")
    synthetic.as_bf16_bits(A)  # still exactly bf16
    s = oracle_mod.colnorm(A)
    srt = np.sort(s)[::-1]
    for k in ks:
        if k < 512:
            assert (srt[k - 1] - srt[k]) / srt[k - 1] >= 1e-3
    changed = np.any(A != case.A, axis=0)
    assert changed.sum() <= touched


def test_generators_are_seeded_and_exact():
    a = synthetic.make_case("c2", scale=dict(n=32, d=64, m=16))
    b = synthetic.make_case("c2", scale=dict(n=32, d=64, m=16))
    assert synthetic.sha256_of(a.A, a.B) == synthetic.sha256_of(b.A, b.B)
    synthetic.as_bf16_bits(a.A)
    synthetic.as_bf16_bits(a.B)
    c1 = synthetic.make_case("c1")
    assert c1.A.shape == (64, 256) and c1.B.shape == (256, 128) and c1.dtype == "f32"
    # chunked drawing gives the same stream as one draw
    rng1 = np.random.Generator(np.random.PCG64(9))
    rng2 = np.random.Generator(np.random.PCG64(9))
    whole = rng1.standard_normal((10, 7))
    parts = np.concatenate([rng2.standard_normal((3, 7)), rng2.standard_normal((7, 7))])
    assert np.array_equal(whole, parts)


def test_round_to_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    r = synthetic.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                  # halfway, even neighbour is 1.0
    assert r[2] == 1.0 + 2 ** -6       # halfway between 1+2^-7 and 1+2^-6: even is 1+2^-6
    assert r[3] == -2.5
    assert np.isfinite(r[4])


def test_gap_fixup_of_the_gated_block(oracle_mod):
    """After enforce_gap_mlp every requested boundary of the oracle's own h
    (gated_mlp's h) has a relative gap of at least 1e-3, and only Wu changed."""
    import synthetic
    from oracle.fixup import enforce_gap_mlp

    c = synthetic.make_mlp_case(dict(n=128, d=256, m=512), seed=3)
    ks = [oracle_mod.k_of(r, 512) for r in (0.5, 0.7)]
    Wu2, touched = enforce_gap_mlp(c.x, c.Wg, c.Wu, 0.8, ks)
    assert touched > 0
    assert np.array_equal(synthetic.round_to_bf16(Wu2), Wu2)
    changed = np.any(Wu2 != c.Wu, axis=0)
    assert 0 < changed.sum() < 512
    res = oracle_mod.gated_mlp(c.x, c.Wg, Wu2, c.Wd, 0.8, 0.5)
    s = np.sort(oracle_mod.colnorm(res.h))[::-1]
    for k in ks:
        assert (s[k - 1] - s[k]) / s[k - 1] >= 1e-3
