"""Pins of the fp64 backward oracle (oracle/grad.py) against facts that do not
come from it.

* finite differences of the C forward oracle (independent code, explicit
  covariance form) against both gradient forms;
* with a zero probe, torch's fp64 autograd of its own softmax attention
  (causal, grouped-query) for dq, dk, dv: textbook attention;
* the probe gradient in closed form: o is linear in rho with slope -Sigma_KV,
  so drho_i = -Sigma^(i)_KV^T dO_i, with Sigma from numpy's weighted
  covariance;
* exact special cases and invariants: one key, identical keys, the effective
  weights summing to one (sum_j dv_j = sum_i dO_i), key-shift invariance
  (sum_j dk_j = 0), linearity in dO;
* the two forms agree.

Each pin takes a namespace holding ``grad_autograd`` and ``grad_expanded``
so that ``test_planted_mistakes_are_caught`` can run the pins against
deliberately broken copies of the oracle source.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import grad as ograd

HERE = os.path.dirname(os.path.abspath(__file__))
GRAD_SRC = os.path.join(os.path.dirname(HERE), "oracle", "grad.py")


def _make(seed, B, Hq, Hkv, T, d, rho_scale=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    rho = rho_scale * rng.standard_normal((B, Hq, T, d))
    dout = rng.standard_normal((B, Hq, T, d))
    return q, k, v, rho, dout


def _both(m, q, k, v, rho, dout, tau):
    return {"autograd": m.grad_autograd(q, k, v, rho, dout, tau),
            "expanded": m.grad_expanded(q, k, v, rho, dout, tau)}


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    return float(np.abs(a - b).max()) <= tol * scale


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

def pin_finite_differences(m):
    """Central differences of sum(dO * o) through the C oracle's explicit form."""
    B, Hq, Hkv, T, d = 1, 4, 2, 6, 5
    tau = 1.0 / math.sqrt(d)
    q, k, v, rho, dout = _make(11, B, Hq, Hkv, T, d)

    def f(q_, k_, v_, r_):
        o = oracle.prefill(q_, k_, v_, r_, tau, form=oracle.EXPLICIT)
        return float((dout * o).sum())

    rng = np.random.default_rng(5)
    h = 1e-6
    forms = _both(m, q, k, v, rho, dout, tau)
    ok = True
    for which, arr in (("q", 0), ("k", 1), ("v", 2), ("rho", 3)):
        base = [q, k, v, rho]
        shape = base[arr].shape
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in shape)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[arr][idx] += h
            minus[arr][idx] -= h
            fd = (f(*plus) - f(*minus)) / (2 * h)
            for name, g in forms.items():
                got = g[arr][idx]
                if abs(got - fd) > 1e-6 * max(1.0, abs(fd)):
                    ok = False
    return ok


def pin_textbook_zero_probe(m):
    """rho = 0: dq, dk, dv equal torch's fp64 autograd of causal GQA softmax attention."""
    B, Hq, Hkv, T, d = 2, 4, 2, 7, 6
    tau = 1.0 / math.sqrt(d)
    q, k, v, _, dout = _make(12, B, Hq, Hkv, T, d)
    rho = np.zeros_like(q)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=True, scale=tau)
    (torch.tensor(dout) * o).sum().backward()
    ref = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
    ok = True
    for g in _both(m, q, k, v, rho, dout, tau).values():
        for got, want in zip(g[:3], ref):
            ok &= _close(got, want, 1e-12)
    return ok


def pin_probe_gradient_closed_form(m):
    """drho_i = -Sigma^(i)_KV^T dO_i, Sigma from numpy's weighted covariance."""
    B, Hq, Hkv, T, d = 1, 2, 1, 6, 4
    tau = 1.0 / math.sqrt(d)
    q, k, v, rho, dout = _make(13, B, Hq, Hkv, T, d)
    want = np.zeros_like(q)
    for h in range(Hq):
        for t in range(T):
            s = tau * (k[0, 0, :t + 1] @ q[0, h, t])
            p = np.exp(s - s.max())
            p /= p.sum()
            if t == 0:
                sigma = np.zeros((d, d))
            else:
                joint = np.concatenate([v[0, 0, :t + 1], k[0, 0, :t + 1]], axis=1)
                sigma = np.cov(joint.T, aweights=p, bias=True)[:d, d:]  # rows v, columns k
            want[0, h, t] = -sigma.T @ dout[0, h, t]
    ok = True
    for g in _both(m, q, k, v, rho, dout, tau).values():
        ok &= _close(g[3], want, 1e-12)
    return ok


def pin_one_key(m):
    """T = 1: o = v_0 whatever q, k, rho: only dv is non-zero, and it is the group's summed dO."""
    B, Hq, Hkv, T, d = 1, 4, 2, 1, 3
    q, k, v, rho, dout = _make(14, B, Hq, Hkv, T, d)
    ok = True
    for g in _both(m, q, k, v, rho, dout, 0.5).values():
        dq, dk, dv, drho = g
        ok &= _close(dq, np.zeros_like(dq), 1e-14) and _close(drho, np.zeros_like(drho), 1e-14)
        ok &= _close(dk, np.zeros_like(dk), 1e-14)
        ok &= _close(dv, dout.reshape(B, Hkv, Hq // Hkv, T, d).sum(axis=2), 1e-14)
    return ok


def pin_identical_keys(m):
    """All keys equal: o is the running mean of v, independent of q and rho."""
    B, Hq, Hkv, T, d = 1, 2, 1, 5, 4
    q, k, v, rho, dout = _make(15, B, Hq, Hkv, T, d)
    k[:] = k[:, :, :1]
    ok = True
    for g in _both(m, q, k, v, rho, dout, 0.7).values():
        ok &= _close(g[0], np.zeros_like(q), 1e-13) and _close(g[3], np.zeros_like(q), 1e-13)
    return ok


def pin_weights_sum_to_one(m):
    """Shifting every value by c shifts o by c: sum_j dv_j = sum over the group's rows of dO."""
    B, Hq, Hkv, T, d = 2, 4, 2, 8, 5
    q, k, v, rho, dout = _make(16, B, Hq, Hkv, T, d, rho_scale=1.5)
    want = dout.reshape(B, Hkv, Hq // Hkv, T, d).sum(axis=(2, 3))
    ok = True
    for g in _both(m, q, k, v, rho, dout, 0.4).values():
        ok &= _close(g[2].sum(axis=2), want, 1e-12)
    return ok


def pin_key_shift_invariance(m):
    """Shifting every key by c leaves o unchanged: sum_j dk_j = 0."""
    B, Hq, Hkv, T, d = 2, 4, 2, 8, 5
    q, k, v, rho, dout = _make(17, B, Hq, Hkv, T, d, rho_scale=1.0)
    ok = True
    for g in _both(m, q, k, v, rho, dout, 0.4).values():
        ok &= _close(g[1].sum(axis=2), np.zeros((B, Hkv, d)), 1e-12)
    return ok


def pin_linear_in_dout(m):
    B, Hq, Hkv, T, d = 1, 2, 2, 6, 4
    q, k, v, rho, d1 = _make(18, B, Hq, Hkv, T, d)
    d2 = np.random.default_rng(19).standard_normal(d1.shape)
    ok = True
    for name in ("grad_autograd", "grad_expanded"):
        fn = getattr(m, name)
        a, b, c = fn(q, k, v, rho, d1, 0.5), fn(q, k, v, rho, d2, 0.5), fn(q, k, v, rho, 2 * d1 - 3 * d2, 0.5)
        for x, y, z in zip(a, b, c):
            ok &= _close(z, 2 * x - 3 * y, 1e-12)
    return ok


def pin_forms_agree(m):
    B, Hq, Hkv, T, d = 2, 4, 2, 9, 6
    q, k, v, rho, dout = _make(20, B, Hq, Hkv, T, d, rho_scale=0.8)
    g = _both(m, q, k, v, rho, dout, 1.0 / math.sqrt(d))
    return all(_close(a, b, 1e-11) for a, b in zip(g["autograd"], g["expanded"]))


PINS = [pin_finite_differences, pin_textbook_zero_probe, pin_probe_gradient_closed_form, pin_one_key,
        pin_identical_keys, pin_weights_sum_to_one, pin_key_shift_invariance, pin_linear_in_dout,
        pin_forms_agree]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_grad_oracle_pin(oracle_mod, pin):
    assert pin(ograd)


def test_grouped_selection_matches_full(oracle_mod):
    q, k, v, rho, dout = _make(21, 2, 4, 2, 7, 3)
    full = ograd.grad_expanded(q, k, v, rho, dout, 0.6)
    part = ograd.grad_expanded(q, k, v, rho, dout, 0.6, groups=[(1, 0), (0, 1)])
    for (b, g), (dq, dk, dv, drho) in part.items():
        assert np.array_equal(dq, full[0][b, 2 * g:2 * g + 2]) and np.array_equal(drho, full[3][b, 2 * g:2 * g + 2])
        assert np.array_equal(dk, full[1][b, g]) and np.array_equal(dv, full[2][b, g])


# --------------------------------------------------------------------------
# forward_stats: the row statistics the training forward keeps (lse2, rbar,
# o^SA), pinned by closed forms, an independent brute force and the C oracle
# --------------------------------------------------------------------------

def fstat_pin_zero_query(m):
    """q = 0: every score is 0, so lse2 = log2(t + 1) exactly and the weights
    are uniform: rbar = mean_j <k_j, rho>, o^SA = mean_j v_j (GQA, Hkv = 2)."""
    B, Hq, Hkv, T, d = 1, 4, 2, 6, 3
    _, k, v, rho, _ = _make(30, B, Hq, Hkv, T, d, rho_scale=1.0)
    q = np.zeros((B, Hq, T, d))
    rows = np.array([[0, h, t] for h in range(Hq) for t in range(T)])
    lse2, rbar, o_sa = m.forward_stats(q, k, v, rho, 0.7, rows)
    ok = True
    for n, (_, h, t) in enumerate(rows):
        kv = h // (Hq // Hkv)
        ok &= abs(lse2[n] - math.log2(t + 1)) < 1e-13
        ok &= abs(rbar[n] - float(np.mean(k[0, kv, :t + 1] @ rho[0, h, t]))) < 1e-13
        ok &= bool(np.abs(o_sa[n] - v[0, kv, :t + 1].mean(axis=0)).max() < 1e-13)
    return ok


def fstat_pin_one_key(m):
    """Row t = 0 has one key: lse2 = s_0 log2 e with s_0 = tau q.k_0,
    rbar = <k_0, rho>, o^SA = v_0."""
    B, Hq, Hkv, T, d = 2, 4, 2, 3, 5
    q, k, v, rho, _ = _make(31, B, Hq, Hkv, T, d)
    tau = 0.45
    rows = np.array([[b, h, 0] for b in range(B) for h in range(Hq)])
    lse2, rbar, o_sa = m.forward_stats(q, k, v, rho, tau, rows)
    ok = True
    for n, (b, h, _) in enumerate(rows):
        k0 = k[b, h // (Hq // Hkv), 0]
        ok &= abs(lse2[n] - tau * float(q[b, h, 0] @ k0) * math.log2(math.e)) < 1e-12
        ok &= abs(rbar[n] - float(rho[b, h, 0] @ k0)) < 1e-12
        ok &= bool(np.abs(o_sa[n] - v[b, h // (Hq // Hkv), 0]).max() < 1e-14)
    return ok


def _brute_stats(q, k, v, rho, tau, b, h, t, G):
    """Plain loops with the math module: lse2, rbar and o^SA of one row."""
    d = len(q[b, h, t])
    g = h // G
    s = [tau * sum(q[b, h, t, a] * k[b, g, j, a] for a in range(d)) for j in range(t + 1)]
    top = max(s)
    e = [math.exp(x - top) for x in s]
    z = sum(e)
    lse2 = (top + math.log(z)) / math.log(2.0)
    r = [sum(rho[b, h, t, a] * k[b, g, j, a] for a in range(d)) for j in range(t + 1)]
    rbar = sum(e[j] / z * r[j] for j in range(t + 1))
    osa = [sum(e[j] / z * v[b, g, j, a] for j in range(t + 1)) for a in range(d)]
    return lse2, rbar, osa


def fstat_pin_brute_force_gqa(m):
    """Every row of a GQA case (Hq = 4, Hkv = 2) against plain loops."""
    B, Hq, Hkv, T, d = 2, 4, 2, 5, 3
    q, k, v, rho, _ = _make(32, B, Hq, Hkv, T, d, rho_scale=0.8)
    tau = 0.6
    rows = np.array([[b, h, t] for b in range(B) for h in range(Hq) for t in range(T)])
    lse2, rbar, o_sa = m.forward_stats(q, k, v, rho, tau, rows)
    ok = True
    for n, (b, h, t) in enumerate(rows):
        l2, rb, osa = _brute_stats(q, k, v, rho, tau, b, h, t, Hq // Hkv)
        ok &= abs(lse2[n] - l2) < 1e-12 and abs(rbar[n] - rb) < 1e-12
        ok &= bool(np.abs(o_sa[n] - np.array(osa)).max() < 1e-12)
    return ok


def fstat_pin_c_oracle_gqa(m):
    """Against the C forward oracle (independent code, GQA with Hkv = 2):
    o^SA is its output with a zero probe, and rbar_i is its softmax output
    for a value column that holds r_j = <rho_i, k_j> (the softmax average of
    r is rbar by definition)."""
    B, Hq, Hkv, T, d = 1, 4, 2, 7, 4
    q, k, v, rho, _ = _make(33, B, Hq, Hkv, T, d)
    rows = np.array([[0, h, t] for h in range(Hq) for t in range(T)])
    lse2, rbar, o_sa = m.forward_stats(q, k, v, rho, 0.5, rows)
    ok = bool(np.abs(o_sa - oracle.prefill(q, k, v, None, 0.5, rows=rows)).max() < 1e-13)
    for n, (_, h, t) in enumerate(rows):
        G = Hq // Hkv
        vr = np.zeros_like(v)
        vr[0, h // G, :, 0] = k[0, h // G] @ rho[0, h, t]
        want = oracle.prefill(q, k, vr, None, 0.5, rows=rows[n:n + 1])[0, 0]
        ok &= abs(rbar[n] - want) < 1e-13
    return ok


FSTAT_PINS = [fstat_pin_zero_query, fstat_pin_one_key, fstat_pin_brute_force_gqa, fstat_pin_c_oracle_gqa]


@pytest.mark.parametrize("pin", FSTAT_PINS, ids=[p.__name__ for p in FSTAT_PINS])
def test_forward_stats_pin(oracle_mod, pin):
    assert pin(ograd)


# --------------------------------------------------------------------------
# planted mistakes: each broken copy of the oracle must fail at least one pin
# --------------------------------------------------------------------------

MUTATIONS = {
    "expanded: sign of D": ("Gs[:, None] * r - D[:, None]", "Gs[:, None] * r + D[:, None]"),
    "expanded: rbar dropped from dS": ("dS = p * (g * (1.0 - r + rbar[:, None])", "dS = p * (g * (1.0 - r)"),
    "expanded: rbar*G dropped from D": ("D = (doh * o).sum(axis=1) + rbar * Gs", "D = (doh * o).sum(axis=1)"),
    "expanded: sign of dR": ("dR = p * (Gs[:, None] - g)", "dR = p * (g - Gs[:, None])"),
    "expanded: probe term dropped from dk": ("dk = tau * (dS.T @ qh) + dR.T @ rh", "dk = tau * (dS.T @ qh)"),
    "expanded: scale dropped from dq": ("dq = tau * (dS @ kh)", "dq = dS @ kh"),
    "expanded: dv from p instead of w": ("dv = w.T @ doh", "dv = p.T @ doh"),
    "autograd: transposed Sigma": ('corr = torch.einsum("tab,tb->ta", sigma, rh)',
                                   'corr = torch.einsum("tba,tb->ta", sigma, rh)'),
    "autograd: sign of the correction": ("o = o_sa - corr", "o = o_sa + corr"),
    "autograd: raw second moment": ("dk_c = kh.unsqueeze(0) - mu_k.unsqueeze(1)", "dk_c = kh.unsqueeze(0) + 0 * mu_k.unsqueeze(1)"),
}


def _mutant(old, new):
    src = open(GRAD_SRC).read()
    if src.count(old) != 1:
        raise AssertionError(f"mutation anchor not found exactly once: {old!r}")
    src = src.replace(old, new)
    if old.startswith("dk_c"):  # the raw second moment needs both factors uncentred
        src = src.replace("dv_c = vh.unsqueeze(0) - o_sa.unsqueeze(1)", "dv_c = vh.unsqueeze(0) + 0 * o_sa.unsqueeze(1)")
    mod = types.ModuleType("grad_mutant")
    exec(compile(src, GRAD_SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistakes_are_caught(oracle_mod, name):
    mod = _mutant(*MUTATIONS[name])
    failed = [p.__name__ for p in PINS if not p(mod)]
    print(f"{name}: caught by {len(failed)} pin(s): {failed}")
    assert failed, f"planted mistake '{name}' passes every pin"


FSTAT_MUTATIONS = {
    "forward_stats: KV head h % Hkv": ("kk = k[b, h // G, :t + 1]", "kk = k[b, h % (q.shape[1] // G), :t + 1]"),
    "forward_stats: natural-log lse": ("lse2[n] = (m + np.log(e.sum())) / np.log(2.0)", "lse2[n] = m + np.log(e.sum())"),
    "forward_stats: unnormalised weights in rbar": ("rbar[n] = p @ (kk @ rho[b, h, t])",
                                                    "rbar[n] = e @ (kk @ rho[b, h, t])"),
    "forward_stats: lse without the max": ("lse2[n] = (m + np.log(e.sum())) / np.log(2.0)",
                                           "lse2[n] = np.log(e.sum()) / np.log(2.0)"),
    "forward_stats: o^SA from the wrong KV head": ("o_sa[n] = p @ v[b, h // G, :t + 1]",
                                                   "o_sa[n] = p @ v[b, (h // G + 1) % (q.shape[1] // G), :t + 1]"),
    "forward_stats: scale dropped": ("s = tau * (kk @ q[b, h, t])", "s = kk @ q[b, h, t]"),
}


@pytest.mark.parametrize("name", list(FSTAT_MUTATIONS))
def test_planted_forward_stats_mistakes_are_caught(oracle_mod, name):
    old, new = FSTAT_MUTATIONS[name]
    src = open(GRAD_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("grad_fstat_mutant")
    exec(compile(src.replace(old, new), GRAD_SRC + " (mutant)", "exec"), mod.__dict__)
    failed = [p.__name__ for p in FSTAT_PINS if not p(mod)]
    print(f"{name}: caught by {len(failed)} pin(s): {failed}")
    assert failed, f"planted mistake '{name}' passes every forward_stats pin"
