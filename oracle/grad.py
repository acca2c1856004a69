"""fp64 CPU oracle of the Parallax attention backward pass (causal prefill).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product library never does.  It
shares no code with the HIP path.

The forward it differentiates is the one the gist.science technical summary of
Parallax gives ("Method: Parallax / core mechanism"): o_i = o^SA_i -
Sigma^(i)_KV rho_i, with the boundary-amplification factor set to zero ("key
design choices"; the news.chathome.org article, "How does the mechanism
work?").  The pages train with this layer (news.chathome.org, "Experiments")
but print no backward pass, so the gradients here are derived, in two
independent ways:

* ``grad_autograd``: torch's reverse-mode differentiation (float64, CPU)
  applied to the explicit definition: per query row the softmax weights p, the
  weighted means of k and v, the d x d covariance matrix built as
  sum_j p_j (v_j - mean v)(k_j - mean k)^T, and o = o^SA - Sigma rho.  Memory
  grows as T^2 d, so it serves small shapes.

* ``grad_expanded``: the closed-form gradients written out by hand, O(T^2 d)
  per head with T x T intermediates.  With r_ij = rho_i . k_j,
  rbar_i = sum_j p_ij r_ij and o^SA_i = sum_j p_ij v_j, the forward is
  o_i = sum_j w_ij v_j with w_ij = p_ij (1 - r_ij + rbar_i).  For an upstream
  gradient dO:

      g_ij = dO_i . v_j           G_i = dO_i . o^SA_i
      D_i  = dO_i . o_i + rbar_i G_i
      dS_ij = p_ij (g_ij (1 - r_ij + rbar_i) + G_i r_ij - D_i)   (w.r.t. s = tau q.k)
      dR_ij = p_ij (G_i - g_ij)                                   (w.r.t. r = rho.k)
      dq_i = tau sum_j dS_ij k_j        drho_i = sum_j dR_ij k_j
      dk_j = tau sum_i dS_ij q_i + sum_i dR_ij rho_i
      dv_j = sum_i w_ij dO_i

  (derivation: dL/dw_ij = g_ij; differentiate w through p, r and rbar, then
  through the softmax.)

Both map causal prefill and GQA the way the forward oracle does: row (b, h, t)
attends keys 0..t of KV head h // G, and the k/v gradients of a KV head sum
over its G query heads.
"""
from __future__ import annotations

import numpy as np


def _check(q, k, v, rho, dout):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, T, d = q.shape
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d) or v.shape != (B, Hkv, T, d):
        raise ValueError("k and v must be [B, Hkv, T, d]")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    rho = np.zeros_like(q) if rho is None else np.asarray(rho, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if rho.shape != q.shape or dout.shape != q.shape:
        raise ValueError("rho and dout must be shaped like q")
    return q, k, v, rho, dout, Hq // Hkv


def grad_autograd(q, k, v, rho, dout, tau: float):
    """Gradients (dq, dk, dv, drho) of sum(dout * o) by torch autograd through
    the explicit covariance form.  Arrays in, float64 numpy arrays out."""
    import torch

    q, k, v, rho, dout, G = _check(q, k, v, rho, dout)
    B, Hq, T, d = q.shape
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    tr = torch.tensor(rho, requires_grad=True)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            qh, rh = tq[b, h], tr[b, h]
            kh, vh = tk[b, h // G], tv[b, h // G]
            s = tau * (qh @ kh.T)
            s = s.masked_fill(~mask, float("-inf"))
            p = torch.softmax(s, dim=-1)                      # [T, T]
            mu_k = p @ kh                                     # [T, d]
            o_sa = p @ vh                                     # [T, d]
            dv_c = vh.unsqueeze(0) - o_sa.unsqueeze(1)        # [T, T, d]: v_j - mean v (row t)
            dk_c = kh.unsqueeze(0) - mu_k.unsqueeze(1)        # [T, T, d]: k_j - mean k (row t)
            sigma = torch.einsum("tj,tja,tjb->tab", p, dv_c, dk_c)  # [T, d(v), d(k)]
            corr = torch.einsum("tab,tb->ta", sigma, rh)
            o = o_sa - corr
            loss = loss + (torch.tensor(dout[b, h]) * o).sum()
    loss.backward()
    return (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), tr.grad.numpy())


def _head_expanded(qh, kh, vh, rh, doh, tau):
    """Closed-form gradients of one query head over its own keys (causal)."""
    T = qh.shape[0]
    s = tau * (qh @ kh.T)
    s[np.triu_indices(T, 1)] = -np.inf
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)                 # [T, T]; zero above the diagonal
    r = rh @ kh.T                                     # [T, T]
    rbar = (p * r).sum(axis=1)                        # [T]
    o_sa = p @ vh
    w = p * (1.0 - r + rbar[:, None])
    o = w @ vh
    g = doh @ vh.T                                    # [T, T]
    Gs = (doh * o_sa).sum(axis=1)
    D = (doh * o).sum(axis=1) + rbar * Gs
    dS = p * (g * (1.0 - r + rbar[:, None]) + Gs[:, None] * r - D[:, None])
    dR = p * (Gs[:, None] - g)
    dq = tau * (dS @ kh)
    drho = dR @ kh
    dk = tau * (dS.T @ qh) + dR.T @ rh
    dv = w.T @ doh
    return dq, dk, dv, drho


def grad_expanded(q, k, v, rho, dout, tau: float, groups=None):
    """Closed-form gradients (dq, dk, dv, drho), float64.

    groups: optional list of (b, g) KV-head groups; then only those groups are
    evaluated and a dict {(b, g): (dq [G, T, d], dk [T, d], dv [T, d],
    drho [G, T, d])} is returned (dq/drho for query heads g*G .. g*G+G-1).
    Without it the full gradients are returned.
    """
    q, k, v, rho, dout, G = _check(q, k, v, rho, dout)
    B, Hq, T, d = q.shape
    Hkv = Hq // G
    sel = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else list(groups)
    res = {}
    for b, g in sel:
        dq = np.zeros((G, T, d))
        drho = np.zeros((G, T, d))
        dk = np.zeros((T, d))
        dv = np.zeros((T, d))
        for i in range(G):
            h = g * G + i
            a, bk, c, e = _head_expanded(q[b, h], k[b, g], v[b, g], rho[b, h], dout[b, h], tau)
            dq[i], drho[i] = a, e
            dk += bk
            dv += c
        res[(b, g)] = (dq, dk, dv, drho)
    if groups is not None:
        return res
    dq = np.zeros_like(q)
    drho = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for (b, g), (a, bk, c, e) in res.items():
        dq[b, g * G:(g + 1) * G] = a
        drho[b, g * G:(g + 1) * G] = e
        dk[b, g] = bk
        dv[b, g] = c
    return dq, dk, dv, drho


def forward_stats(q, k, v, rho, tau: float, rows):
    """Per-row quantities a training forward keeps for the backward: the
    log2-sum-exp of the scaled scores (lse2 = log2 sum_j 2^(s_ij log2 e)),
    rbar_i and o^SA_i, for the rows (b, h, t) given as an [n, 3] array."""
    q, k, v, rho, _, G = _check(q, k, v, rho, np.zeros_like(np.asarray(q, dtype=np.float64)))
    sel = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    d = q.shape[3]
    lse2 = np.zeros(len(sel))
    rbar = np.zeros(len(sel))
    o_sa = np.zeros((len(sel), d))
    for n, (b, h, t) in enumerate(sel):
        kk = k[b, h // G, :t + 1]
        s = tau * (kk @ q[b, h, t])
        m = s.max()
        e = np.exp(s - m)
        lse2[n] = (m + np.log(e.sum())) / np.log(2.0)
        p = e / e.sum()
        rbar[n] = p @ (kk @ rho[b, h, t])
        o_sa[n] = p @ v[b, h // G, :t + 1]
    return lse2, rbar, o_sa
