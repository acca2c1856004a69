"""Helpers for the GPU parity tests: tolerances, error metrics, and moving
device tensors to the host for the oracle."""
import sys

import numpy as np
import torch

# Tolerances of the method's acceptance bar: fp32 max-abs 1e-5; bf16 max-abs
# 2e-2 and relative L2 5e-3, both against the fp64 oracle on the same rounded
# inputs.
TOL = {torch.float32: dict(max_abs=1e-5, rel_l2=None), torch.bfloat16: dict(max_abs=2e-2, rel_l2=5e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a device tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got.astype(np.float64) - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel()) / denom) if denom > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel


def assert_close(got: np.ndarray, ref: np.ndarray, dtype, what: str):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    tol = TOL[dtype]
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if got.size:
        i = np.unravel_index(int(np.abs(got - ref).argmax()), got.shape)
        say(f"    worst element at {tuple(int(j) for j in i)}: got {got[i]!r} oracle {ref[i]!r}; "
            f"max |oracle| {float(np.abs(ref).max()):.3f}")
    assert max_abs <= tol["max_abs"], f"{what}: max_abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: rel_l2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits, round to nearest even)
U_F32 = 2.0 ** -24


def _rows_bound(Q, Rh, K, V, mask, tau, dtype, n_merge=1):
    """First-order rounding bound, per element, for query rows Q (probes Rh)
    over keys K, values V (mask[i, j]: key j is in row i's context).

    The kernels form P_j = 2^(s_j log2e - m) in fp32, round P_j and P_j r_j to
    the matrix-core operand type, take l and c over the rounded operands, and
    finish o = A/l - (B/l - (c/l) A/l).  With w_j the exact softmax weights,
    z_j = w_j r_j, relative operand errors eps_j (of P_j) and eta_j (of
    P_j r_j) and absolute errors dr_j of r_j, the weights that multiply V sum
    to one exactly, and to first order

        o_gpu - o = (1 + cbar) sum_j w_j eps_j (v_j - o^SA)
                    - sum_j (z_j (eta_j - epsbar) + w_j dr_j) (v_j - o^SA)

    with epsbar = sum_j w_j eps_j, plus the output's own rounding.  eps_j holds
    the fp32 errors of the score (d-term accumulation), of the exponent
    argument and of exp2, plus the operand rounding (bf16 only: fp32 operands
    are used as they are).  A slack for the fp32 accumulation over the keys
    and the rescales is added.  n_merge > 1 adds the merge's exp2 per chunk.
    """
    n, d = Q.shape
    L = K.shape[0]
    bf = dtype == torch.bfloat16
    u_op = U_BF16 if bf else 0.0
    u_pr = U_BF16 if bf else U_F32
    u_out = U_BF16 if bf else U_F32
    S = tau * (Q @ K.T)
    S = np.where(mask, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.where(mask, np.exp(np.where(mask, S, 0.0) - m), 0.0)
    tot = E.sum(axis=1, keepdims=True)
    W = E / np.where(tot > 0, tot, 1.0)
    R = Rh @ K.T
    Z = W * R
    osa = W @ V
    cbar = Z.sum(axis=1)
    o = osa - (Z @ V - cbar[:, None] * osa)
    Sf = np.where(mask, np.abs(S), 0.0)
    eps32 = (tau * d * U_F32 * (np.abs(Q) @ np.abs(K).T) + U_F32 * (2 * Sf + np.abs(m))
             + 2 * U_F32 * (1 + n_merge))
    eps = eps32 + u_op
    eta = eps32 + u_pr
    dr = d * U_F32 * (np.abs(Rh) @ np.abs(K).T)
    epsbar = (W * eps).sum(axis=1, keepdims=True)
    coef = np.abs(1 + cbar)[:, None] * W * eps + np.abs(Z) * (eta + epsbar) + W * dr
    out = np.empty((n, d))
    for i0 in range(0, n, 32):
        dev = np.abs(V[None, :, :] - osa[i0:i0 + 32, None, :])
        out[i0:i0 + 32] = np.einsum("nl,nld->nd", coef[i0:i0 + 32], dev)
    acc = (L / 16 + 64) * U_F32 * (((W + np.abs(Z)) @ np.abs(V)) * (1 + np.abs(cbar))[:, None])
    # The output rounds the kernel's value y, not o: |fl(y) - o| <= u|o| + (1 + u)|y - o|.
    return (out + acc) * (1 + u_out) + u_out * np.abs(o)


def bound_prefill(q, k, v, rho, tau, dtype):
    """Per-element rounding bound of a causal prefill ([B, Hq, T, d])."""
    B, Hq, T, d = q.shape
    G = Hq // k.shape[1]
    rho = np.zeros_like(q) if rho is None else rho
    mask = np.tril(np.ones((T, T), dtype=bool))
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = _rows_bound(q[b, h], rho[b, h], k[b, h // G], v[b, h // G], mask, tau, dtype)
    return out


def bound_decode(q, rho, k, v, tau, dtype, cu_seqlens=None, Hkv=None, n_merge=1):
    """Per-element rounding bound of a decode ([B, Hq, d]); cache as in the
    oracle's decode (contiguous [B, Hkv, L, d], or packed slabs + cu_seqlens)."""
    B, Hq, d = q.shape
    rho = np.zeros_like(q) if rho is None else rho
    out = np.zeros_like(q)
    for b in range(B):
        if cu_seqlens is None:
            kb, vb = k[b], v[b]
        else:
            L = int(cu_seqlens[b + 1] - cu_seqlens[b])
            s0 = int(cu_seqlens[b]) * Hkv * d
            kb = k.reshape(-1)[s0:s0 + Hkv * L * d].reshape(Hkv, L, d)
            vb = v.reshape(-1)[s0:s0 + Hkv * L * d].reshape(Hkv, L, d)
        if kb.shape[1] == 0:
            continue
        G = Hq // kb.shape[0]
        mask = np.ones((1, kb.shape[1]), dtype=bool)
        for h in range(Hq):
            out[b, h] = _rows_bound(q[b, h][None], rho[b, h][None], kb[h // G], vb[h // G], mask, tau, dtype,
                                    n_merge)[0]
    return out


def assert_within_bound(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str, rel_l2=5e-3):
    """Every element within its derived rounding bound (see _rows_bound), and
    rel-L2 at most 5e-3.  For inputs whose outputs are O(1) (sharp weights,
    contexts of a few keys) the fixed max-abs bar of the workloads cannot hold
    by construction: an output near 6 has a bf16 spacing of 2^-5."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs, rel = errors(got, ref)
    ratio = err / np.maximum(bound, 1e-300)
    i = np.unravel_index(int(ratio.argmax()), ratio.shape) if ratio.size else ()
    say(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst err/bound={float(ratio.max()) if ratio.size else 0:.3f}"
        + (f" at {tuple(int(j) for j in i)} (err {float(err[i]):.3e}, bound {float(bound[i]):.3e}, "
           f"oracle {float(ref[i]):.4f})" if ratio.size else ""))
    assert (err <= bound).all(), f"{what}: {int((err > bound).sum())} elements beyond their rounding bound"
    assert rel <= rel_l2, f"{what}: rel_l2 {rel:.3e}"


def gpu_available() -> bool:
    return torch.cuda.is_available()
