"""Pins of the projection oracle (oracle/projection.py): a one-hot token picks
out one column of the weight in the stated place; the matmul form equals a
nested-loop brute force of the indexing; and linearity."""
import numpy as np
import pytest

from oracle import projection as proj


def test_one_hot_token_selects_weight_columns():
    Hq, Hkv, d, dm = 4, 2, 3, 5
    rng = np.random.default_rng(0)
    w = rng.standard_normal((sum(proj.feature_counts(Hq, Hkv, d)), dm))
    x = np.zeros((2, 3, dm))
    x[1, 2, 4] = 1.0                       # token (b=1, t=2) is the unit vector e_4
    q, k, v, r = proj.project(x, w, Hq, Hkv, d)
    offs = np.cumsum((0,) + proj.feature_counts(Hq, Hkv, d))
    for out, off, H in zip((q, k, v, r), offs, (Hq, Hkv, Hkv, Hq)):
        for h in range(H):
            assert np.array_equal(out[1, h, 2], w[off + h * d: off + (h + 1) * d, 4])
        mask = np.ones(out.shape, dtype=bool)
        mask[1, :, 2] = False
        assert not out[mask].any()         # every other token projects to zero


def test_matmul_form_equals_brute_force():
    Hq, Hkv, d, dm = 4, 2, 3, 7
    rng = np.random.default_rng(1)
    w = rng.standard_normal((sum(proj.feature_counts(Hq, Hkv, d)), dm))
    x = rng.standard_normal((2, 5, dm))
    for a, b in zip(proj.project(x, w, Hq, Hkv, d), proj.project_loops(x, w, Hq, Hkv, d)):
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_linear_in_x_and_w():
    Hq, Hkv, d, dm = 2, 1, 4, 6
    rng = np.random.default_rng(2)
    w1, w2 = (rng.standard_normal((sum(proj.feature_counts(Hq, Hkv, d)), dm)) for _ in range(2))
    x1, x2 = (rng.standard_normal((1, 3, dm)) for _ in range(2))
    for a, b, c in zip(proj.project(2 * x1 - x2, w1, Hq, Hkv, d), proj.project(x1, w1, Hq, Hkv, d),
                       proj.project(x2, w1, Hq, Hkv, d)):
        assert np.allclose(a, 2 * b - c, atol=1e-12)
    for a, b, c in zip(proj.project(x1, w1 + 3 * w2, Hq, Hkv, d), proj.project(x1, w1, Hq, Hkv, d),
                       proj.project(x1, w2, Hq, Hkv, d)):
        assert np.allclose(a, b + 3 * c, atol=1e-12)


# Planted mistakes in the matmul form: each must fail at least one pin.
MUTATIONS = {
    "no_head_major_transpose": ("part.reshape(B, T, H, d).transpose(0, 2, 1, 3).copy()",
                                "part.reshape(B, H, T, d).copy()"),
    "head_and_dim_swapped": ("part.reshape(B, T, H, d).transpose(0, 2, 1, 3).copy()",
                             "part.reshape(B, T, d, H).transpose(0, 3, 1, 2).copy()"),
    "blocks_shifted": ("part = y[:, start:start + n_feat]", "part = np.roll(y, 1, axis=1)[:, start:start + n_feat]"),
    "weight_scaled": ("y = x.reshape(B * T, dm) @ w.T", "y = x.reshape(B * T, dm) @ (0.5 * w.T)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    import inspect
    import types
    src = inspect.getsource(proj)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor not unique: {old}"
    mutant = types.ModuleType("projection_mutant")
    exec(compile(src.replace(old, new), "projection_mutant", "exec"), mutant.__dict__)
    # the pins read proj.project; the brute force stays the original
    monkeypatch.setattr(proj, "project", mutant.project)
    caught = []
    for pin in (test_one_hot_token_selects_weight_columns, test_matmul_form_equals_brute_force, test_linear_in_x_and_w):
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
