"""fp64 CPU oracle of the fused probe projection.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product library never does.  It
shares no code with the HIP path.

The probe is a learned linear map of the layer input, rho_i = W_R x_i (the
news.chathome.org article, "What is Parallax"; the gist.science summary,
"Method: Parallax / core mechanism"), computed beside the usual q, k and v
projections.  One weight matrix stacks the four projections by output
feature: rows 0 .. Hq*d-1 give q (head-major: feature h*d + a is dim a of
query head h), then Hkv*d rows for k, Hkv*d for v, and Hq*d for rho (one probe
per query head).  There is no bias (the pages give none).  For tokens
x [B, T, d_model] the outputs are laid out as the attention kernels read
them: q, rho [B, Hq, T, d]; k, v [B, Hkv, T, d].

The product itself is a library matmul in float64 on the exactly upcast
inputs; the rest is the split by feature ranges and the head-major
transpose, written out plainly.
"""
from __future__ import annotations

import numpy as np


def feature_counts(Hq: int, Hkv: int, d: int):
    """(q, k, v, rho) output-feature counts, in stacking order."""
    return (Hq * d, Hkv * d, Hkv * d, Hq * d)


def project(x, w, Hq: int, Hkv: int, d: int):
    """x: [B, T, d_model]; w: [(2 Hq + 2 Hkv) d, d_model] (one row per output
    feature, as a torch Linear weight).  Returns (q, k, v, rho) float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, dm = x.shape
    counts = feature_counts(Hq, Hkv, d)
    if w.shape != (sum(counts), dm):
        raise ValueError("w must be [(2 Hq + 2 Hkv) d, d_model]")
    y = x.reshape(B * T, dm) @ w.T                      # [B*T, features]
    outs = []
    start = 0
    for n_feat in counts:
        part = y[:, start:start + n_feat]
        start += n_feat
        H = n_feat // d
        # feature h*d + a of token (b, t) -> [b, h, t, a]
        outs.append(part.reshape(B, T, H, d).transpose(0, 2, 1, 3).copy())
    return tuple(outs)


def project_loops(x, w, Hq: int, Hkv: int, d: int):
    """The same map as nested Python loops (tiny sizes only): a brute-force
    statement of the indexing."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, dm = x.shape
    shapes = [(B, Hq, T, d), (B, Hkv, T, d), (B, Hkv, T, d), (B, Hq, T, d)]
    outs = [np.zeros(s) for s in shapes]
    n = 0
    for which, (_, H, _, _) in enumerate(shapes):
        for h in range(H):
            for a in range(d):
                for b in range(B):
                    for t in range(T):
                        acc = 0.0
                        for c in range(dm):
                            acc += w[n, c] * x[b, t, c]
                        outs[which][b, h, t, a] = acc
                n += 1
    return tuple(outs)
