"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each pin ties the oracle to something fixed by the pages or by mathematics:
a hand-worked example (tests/golden), exact special cases, invariants, a
textbook special case computed by a library routine (torch's fp64 softmax
attention, numpy's weighted covariance), exact rational arithmetic, and a
pure-Python brute force of the causal / GQA / ragged index mapping.

The pins are written as functions of the loaded C library so that
``test_planted_mistakes_are_caught`` can run them against deliberately broken
copies of the oracle source: every planted mistake must fail at least one pin.
"""
import json
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _frac(s):
    return float(Fraction(s))


def _rows(lib, q, rho, K, V, tau, form):
    """One query row over K, V ([L, d]) through the oracle's row interface."""
    q = np.asarray(q, dtype=np.float64)[None, :]
    r = None if rho is None else np.asarray(rho, dtype=np.float64)[None, :]
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    return oracle.attend_rows(q, r, K, V, [0], [K.shape[0]], K.shape[1], tau, form, lib=lib)[0]


FORMS = (oracle.EXPLICIT, oracle.EXPANDED)


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

def pin_hand_example(lib):
    """W: hand-worked two-key, d = 2 example (tests/golden)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example_2key_d2.json")))
    tau = 1.0 / math.sqrt(2.0)
    q = [math.log(3.0) / math.sqrt(2.0), 0.0]
    K = [[_frac(x) for x in row] for row in g["k"]]
    V = [[_frac(x) for x in row] for row in g["v"]]
    for case in g["cases"]:
        rho = [_frac(x) for x in case["rho"]]
        want = np.array([_frac(x) for x in case["o"]])
        for form in FORMS:
            got = _rows(lib, q, rho, K, V, tau, form)
            assert np.allclose(got, want, rtol=0, atol=1e-14), (case, form, got)
    # the same tokens as a causal sequence: row 0 sees only key 0
    qq = np.array([[[[0.3, -0.7], q]]])  # [1, 1, 2, 2]; row 0's q is arbitrary
    rr = np.array([[[[1.0, 0.0], [1.0, 0.0]]]])
    kk = np.array([[K]])
    vv = np.array([[V]])
    for form in FORMS:
        out = oracle.prefill(qq, kk, vv, rr, tau, form=form, lib=lib)
        assert np.allclose(out[0, 0, 0], [_frac(x) for x in g["causal_T2"]["o_t0"]], atol=1e-15)
        assert np.allclose(out[0, 0, 1], [_frac(x) for x in g["causal_T2"]["o_t1"]], atol=1e-14)


def pin_rho_zero_is_softmax_attention(lib):
    """I1 + L1: a zero probe gives plain softmax attention, checked against
    torch's fp64 CPU scaled_dot_product_attention (causal, GQA) and with the
    probe omitted; the correction vanishes exactly."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, T, d = 2, 4, 2, 9, 8
    tau = 0.37
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, scale=tau, enable_gqa=True).numpy()
    for form in FORMS:
        none = oracle.prefill(q, k, v, None, tau, form=form, lib=lib)
        zero = oracle.prefill(q, k, v, np.zeros_like(q), tau, form=form, lib=lib)
        assert np.array_equal(none, zero), form
        assert np.abs(none - ref).max() < 1e-12, form
    # decode over a contiguous cache: every query attends all L keys
    L = 7
    qd = rng.standard_normal((B, Hq, d))
    kd = rng.standard_normal((B, Hkv, L, d))
    vd = rng.standard_normal((B, Hkv, L, d))
    refd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qd)[:, :, None, :], torch.from_numpy(kd), torch.from_numpy(vd),
        scale=tau, enable_gqa=True).numpy()[:, :, 0, :]
    for form in FORMS:
        got = oracle.decode(qd, np.zeros_like(qd), kd, vd, tau, form=form, lib=lib)
        assert np.abs(got - refd).max() < 1e-12, form


def pin_one_key(lib):
    """I2: a single key gives weight 1, zero covariance, o = v_0."""
    rng = np.random.default_rng(12)
    for d in (1, 4, 16):
        q, rho, k, v = (rng.standard_normal(d) for _ in range(4))
        for form in FORMS:
            got = _rows(lib, q, rho * 5, k[None], v[None], 0.9, form)
            assert np.allclose(got, v, rtol=0, atol=1e-15), (d, form)


def pin_identical_keys(lib):
    """I3: identical keys centre to zero, so no correction, and the weights
    are uniform: o = mean of the values for any probe."""
    rng = np.random.default_rng(13)
    L, d = 6, 5
    k = np.tile(rng.standard_normal(d), (L, 1))
    v = rng.standard_normal((L, d))
    for form in FORMS:
        got = _rows(lib, rng.standard_normal(d), 3 * rng.standard_normal(d), k, v, 0.7, form)
        assert np.allclose(got, v.mean(axis=0), rtol=0, atol=1e-14), form


def pin_constant_values(lib):
    """I4: equal values have zero covariance with anything and the weights
    sum to one, so o = that value."""
    rng = np.random.default_rng(14)
    L, d = 9, 4
    c = rng.standard_normal(d)
    for form in FORMS:
        got = _rows(lib, rng.standard_normal(d), 4 * rng.standard_normal(d),
                    rng.standard_normal((L, d)), np.tile(c, (L, 1)), 0.5, form)
        assert np.allclose(got, c, rtol=0, atol=1e-14), form


def pin_effective_weights(lib):
    """I5 (news.chathome.org article, 'Score differences': per-token weights
    can be negative and exceed 1).  The output is linear in the values, so
    values set to unit vectors read the effective weight of each key off the
    output.  They must sum to 1, equal p_j (1 - r_j + rbar) with p from
    torch's fp64 softmax, and, for a large enough probe, leave [0, 1]."""
    rng = np.random.default_rng(15)
    L, d, tau = 6, 8, 0.4
    q = rng.standard_normal(d)
    k = rng.standard_normal((L, d))
    V = np.eye(d)[:L]
    for scale in (0.1, 3.0):
        rho = scale * rng.standard_normal(d)
        p = torch.softmax(torch.from_numpy(tau * (k @ q)), dim=0).numpy()
        r = k @ rho
        want = p * (1.0 - r + p @ r)
        for form in FORMS:
            w = _rows(lib, q, rho, k, V, tau, form)[:L]
            assert abs(w.sum() - 1.0) < 1e-13, form
            assert np.allclose(w, want, rtol=0, atol=1e-13), form
            if scale > 1:
                assert w.min() < 0 and w.max() > 1, w


def pin_linear_in_probe(lib):
    """I6: the correction o^SA - o is linear in rho (no hidden scale or
    offset on the probe branch)."""
    rng = np.random.default_rng(16)
    L, d, tau = 11, 6, 0.6
    q, k, v = rng.standard_normal(d), rng.standard_normal((L, d)), rng.standard_normal((L, d))
    r1, r2 = rng.standard_normal(d), rng.standard_normal(d)
    for form in FORMS:
        osa = _rows(lib, q, None, k, v, tau, form)
        c1 = osa - _rows(lib, q, r1, k, v, tau, form)
        c2 = osa - _rows(lib, q, r2, k, v, tau, form)
        c3 = osa - _rows(lib, q, 2.5 * r1 - r2, k, v, tau, form)
        assert np.allclose(c3, 2.5 * c1 - c2, rtol=0, atol=1e-13), form
        assert np.abs(c1).max() > 1e-3


def pin_shift_invariance(lib):
    """I7: shifting every key by t shifts every score of a row by the same
    amount and leaves the centred keys alone, so o is unchanged; shifting
    every value by t shifts o by t."""
    rng = np.random.default_rng(17)
    L, d, tau = 10, 5, 0.45
    q, rho = rng.standard_normal(d), rng.standard_normal(d)
    k, v = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    t = rng.standard_normal(d)
    for form in FORMS:
        base = _rows(lib, q, rho, k, v, tau, form)
        assert np.allclose(_rows(lib, q, rho, k + t, v, tau, form), base, rtol=0, atol=1e-13)
        assert np.allclose(_rows(lib, q, rho, k, v + t, tau, form), base + t, rtol=0, atol=1e-13)


def pin_forms_agree(lib):
    """I8: the explicit d x d covariance form and the expanded O(L d) form
    agree on random inputs (prefill with GQA, ragged decode)."""
    rng = np.random.default_rng(18)
    B, Hq, Hkv, T, d = 2, 6, 3, 13, 8
    q = rng.standard_normal((B, Hq, T, d))
    rho = 0.5 * rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    a = oracle.prefill(q, k, v, rho, 0.3, form=oracle.EXPLICIT, lib=lib)
    b = oracle.prefill(q, k, v, rho, 0.3, form=oracle.EXPANDED, lib=lib)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())
    lens = np.array([5, 0, 16, 1])
    cu = np.concatenate([[0], np.cumsum(lens)])
    kf = rng.standard_normal(int(cu[-1]) * Hkv * d)
    vf = rng.standard_normal(int(cu[-1]) * Hkv * d)
    qd = rng.standard_normal((4, Hq, d))
    rd = rng.standard_normal((4, Hq, d))
    a = oracle.decode(qd, rd, kf, vf, 0.3, cu_seqlens=cu, Hkv=Hkv, form=oracle.EXPLICIT, lib=lib)
    b = oracle.decode(qd, rd, kf, vf, 0.3, cu_seqlens=cu, Hkv=Hkv, form=oracle.EXPANDED, lib=lib)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def pin_weighted_covariance_library(lib):
    """L2: Sigma_KV is numpy's weighted population covariance of the stacked
    (value, key) samples with the softmax weights; o = o^SA - Sigma_KV rho
    with o^SA and the weights from torch's fp64 softmax."""
    rng = np.random.default_rng(19)
    L, d, tau = 12, 6, 0.5
    q, rho = rng.standard_normal(d), rng.standard_normal(d)
    k, v = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    p = torch.softmax(torch.from_numpy(tau * (k @ q)), dim=0).numpy()
    sigma = np.cov(np.hstack([v, k]).T, aweights=p, bias=True)[:d, d:]
    want = p @ v - sigma @ rho
    for form in FORMS:
        got = _rows(lib, q, rho, k, v, tau, form)
        assert np.allclose(got, want, rtol=0, atol=1e-13), form


def _exact_uniform(rho, K, V):
    """Exact rational Parallax output for uniform weights (q = 0)."""
    L, d = len(K), len(K[0])
    p = Fraction(1, L)
    mu_k = [sum(p * K[j][b] for j in range(L)) for b in range(d)]
    mu_v = [sum(p * V[j][a] for j in range(L)) for a in range(d)]
    out = []
    for a in range(d):
        corr = Fraction(0)
        for b in range(d):
            cov = sum(p * (V[j][a] - mu_v[a]) * (K[j][b] - mu_k[b]) for j in range(L))
            corr += cov * rho[b]
        out.append(mu_v[a] - corr)
    return out


def pin_exact_rational(lib):
    """L3: with q = 0 every weight is exactly 1/L and the whole result is
    rational; small dyadic inputs make fp64 inputs exact, so the oracle must
    match exact arithmetic to within fp64 rounding."""
    rng = np.random.default_rng(20)
    for d, L in ((1, 2), (2, 3), (3, 5), (3, 6)):
        K = [[Fraction(int(x), 8) for x in rng.integers(-16, 17, d)] for _ in range(L)]
        V = [[Fraction(int(x), 4) for x in rng.integers(-8, 9, d)] for _ in range(L)]
        rho = [Fraction(int(x), 2) for x in rng.integers(-4, 5, d)]
        want = np.array([float(x) for x in _exact_uniform(rho, K, V)])
        for form in FORMS:
            got = _rows(lib, np.zeros(d), [float(x) for x in rho],
                        [[float(x) for x in r] for r in K], [[float(x) for x in r] for r in V],
                        1.3, form)
            assert np.allclose(got, want, rtol=1e-15, atol=1e-15), (d, L, form, got, want)


def _brute_row(q, rho, keys, vals, tau):
    """Pure-Python Parallax row from the definition (nested lists, math.exp)."""
    if not keys:
        return [0.0] * len(q)
    d = len(q)
    s = [tau * sum(q[a] * kk[a] for a in range(d)) for kk in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = sum(w)
    p = [x / z for x in w]
    mk = [sum(p[j] * keys[j][b] for j in range(len(keys))) for b in range(d)]
    mv = [sum(p[j] * vals[j][a] for j in range(len(keys))) for a in range(d)]
    out = []
    for a in range(d):
        c = 0.0
        for b in range(d):
            c += sum(p[j] * (vals[j][a] - mv[a]) * (keys[j][b] - mk[b])
                     for j in range(len(keys))) * rho[b]
        out.append(mv[a] - c)
    return out


def pin_bruteforce_layouts(lib, mod=oracle):
    """Pure-Python loops over nested per-sequence lists check the index
    mapping: causal keys 0..t with the diagonal, query head h on KV head
    h // G, packed ragged slabs (including an empty sequence: output 0), and
    the contiguous cache [B, Hkv, L, d].  `mod` is the oracle module (the
    planted-mistake test passes broken copies of it)."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, T, d, tau = 2, 4, 2, 5, 3, 0.8
    G = Hq // Hkv
    q = rng.standard_normal((B, Hq, T, d))
    rho = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    for form in FORMS:
        got = mod.prefill(q, k, v, rho, tau, form=form, lib=lib)
        for b in range(B):
            for h in range(Hq):
                for t in range(T):
                    keys = [list(k[b, h // G, j]) for j in range(t + 1)]
                    vals = [list(v[b, h // G, j]) for j in range(t + 1)]
                    want = _brute_row(list(q[b, h, t]), list(rho[b, h, t]), keys, vals, tau)
                    assert np.allclose(got[b, h, t], want, rtol=0, atol=1e-12), (b, h, t, form)
    # ragged decode: sequences as separate [Hkv, L_b, d] arrays, then packed
    lens = [3, 0, 1, 6]
    seqs_k = [rng.standard_normal((Hkv, n, d)) for n in lens]
    seqs_v = [rng.standard_normal((Hkv, n, d)) for n in lens]
    packed_k = np.concatenate([s.ravel() for s in seqs_k])
    packed_v = np.concatenate([s.ravel() for s in seqs_v])
    cu = np.concatenate([[0], np.cumsum(lens)])
    qd = rng.standard_normal((len(lens), Hq, d))
    rd = rng.standard_normal((len(lens), Hq, d))
    for form in FORMS:
        got = mod.decode(qd, rd, packed_k, packed_v, tau, cu_seqlens=cu, Hkv=Hkv,
                         form=form, lib=lib)
        for b, n in enumerate(lens):
            for h in range(Hq):
                keys = [list(seqs_k[b][h // G, j]) for j in range(n)]
                vals = [list(seqs_v[b][h // G, j]) for j in range(n)]
                want = _brute_row(list(qd[b, h]), list(rd[b, h]), keys, vals, tau)
                assert np.allclose(got[b, h], want, rtol=0, atol=1e-12), (b, h, form)
    # contiguous decode cache: every sequence has all L keys of its own [Hkv, L, d] block
    L = 4
    kc = rng.standard_normal((len(lens), Hkv, L, d))
    vc = rng.standard_normal((len(lens), Hkv, L, d))
    for form in FORMS:
        got = mod.decode(qd, rd, kc, vc, tau, form=form, lib=lib)
        for b in range(len(lens)):
            for h in range(Hq):
                want = _brute_row(list(qd[b, h]), list(rd[b, h]), [list(x) for x in kc[b, h // G]],
                                  [list(x) for x in vc[b, h // G]], tau)
                assert np.allclose(got[b, h], want, rtol=0, atol=1e-12), (b, h, form, "contiguous")


PINS = [pin_hand_example, pin_rho_zero_is_softmax_attention, pin_one_key,
        pin_identical_keys, pin_constant_values, pin_effective_weights,
        pin_linear_in_probe, pin_shift_invariance, pin_forms_agree,
        pin_weighted_covariance_library, pin_exact_rational, pin_bruteforce_layouts]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(oracle_mod, pin):
    pin(None)


# --------------------------------------------------------------------------
# planted mistakes: each textual change to a copy of the oracle source must
# make at least one pin fail
# --------------------------------------------------------------------------

MUTATIONS = {
    "explicit_sign_of_correction": ("out[a] = mu_v[a] - corr;", "out[a] = mu_v[a] + corr;"),
    "expanded_sign_of_correction": ("out[a] = osa[a] - (prv[a] - rbar * osa[a]);",
                                    "out[a] = osa[a] + (prv[a] - rbar * osa[a]);"),
    "expanded_dropped_mean_term": ("out[a] = osa[a] - (prv[a] - rbar * osa[a]);",
                                   "out[a] = osa[a] - prv[a];"),
    "explicit_transposed_covariance": ("corr += sigma[(size_t)a * d + b] * rho[b];",
                                       "corr += sigma[(size_t)b * d + a] * rho[b];"),
    "expanded_scale_on_probe_scores": ("r[j] = rk;", "r[j] = tau * rk;"),
    # centring only one factor is harmless (the other's weighted deviations
    # sum to zero); dropping both centrings gives the raw second moment
    "explicit_raw_second_moment": ("double dv = p[j] * (vj[a] - mu_v[a]);\n            for (b = 0; b < d; ++b) sigma[(size_t)a * d + b] += dv * (kj[b] - mu_k[b]);",
                                   "double dv = p[j] * vj[a];\n            for (b = 0; b < d; ++b) sigma[(size_t)a * d + b] += dv * kj[b];"),
    "explicit_scale_missing": ("s *= tau;", "s *= 1.0;"),
    "expanded_weights_not_normalised": ("double pj = w[j] / total;", "double pj = w[j];"),
    "explicit_bessel_correction": ("for (j = 0; j < L; ++j) p[j] /= z;",
                                   "for (j = 0; j < L; ++j) p[j] /= z * (L > 1 ? (L - 1.0) / L : 1.0);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_mod, tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "parallax_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old}"
    path_c = tmp_path / "mutant.c"
    path_so = tmp_path / "libmutant.so"
    path_c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o",
                    str(path_so), str(path_c), "-lm"], check=True)
    lib = oracle.load_variant(str(path_so))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


def test_empty_context_reads_no_key(oracle_mod):
    """A sequence with no key returns zeros, and its bounds check looks at no
    storage: a batch of empty ragged sequences needs none at all."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 4, 64))
    rho = 0.1 * rng.standard_normal((3, 4, 64))
    none = np.zeros(1)
    out = oracle.decode(q, rho, none, none, 0.125, cu_seqlens=np.zeros(4, dtype=np.int64), Hkv=2)
    assert out.shape == q.shape and not out.any()
    # one non-empty sequence among empty ones still has to fit its storage
    kv = rng.standard_normal(2 * 5 * 64)
    out = oracle.decode(q, rho, kv, kv, 0.125, cu_seqlens=np.array([0, 0, 5, 5]), Hkv=2)
    assert not out[0].any() and not out[2].any() and np.abs(out[1]).max() > 0
    with pytest.raises(ValueError):
        oracle.decode(q, rho, kv[:-1], kv[:-1], 0.125, cu_seqlens=np.array([0, 0, 5, 5]), Hkv=2)


# Planted mistakes in the Python half of the oracle (the index mapping onto
# rows): each must make the brute-force layout pin fail.
PY_MUTATIONS = {
    "prefill_gqa_interleaved": ("key_off = ((b * Hkv + h // G) * T) * d", "key_off = ((b * Hkv + h % Hkv) * T) * d"),
    "prefill_diagonal_dropped": ("key_len = t + 1", "key_len = np.maximum(t, 1)"),
    "decode_gqa_interleaved": ("key_off = (starts[b] * Hkv + (h // G) * lens[b]) * d",
                               "key_off = (starts[b] * Hkv + (h % Hkv) * lens[b]) * d"),
    "decode_slab_start_per_token": ("key_off = (starts[b] * Hkv + (h // G) * lens[b]) * d",
                                    "key_off = (starts[b] + (h // G) * lens[b]) * d"),
    "decode_contiguous_stride": ("starts = np.arange(B, dtype=np.int64) * L", "starts = np.arange(B, dtype=np.int64) * (L - 1)"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_planted_python_mapping_mistakes_are_caught(oracle_mod, name):
    import types
    path = oracle.__file__
    src = open(path).read()
    old, new = PY_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old}"
    mutant = types.ModuleType("oracle_mutant")
    mutant.__file__ = path  # the mutant loads the real C library next to it
    exec(compile(src.replace(old, new), path, "exec"), mutant.__dict__)
    with pytest.raises((AssertionError, ValueError)):
        pin_bruteforce_layouts(None, mod=mutant)
