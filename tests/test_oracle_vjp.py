"""Pins for the oracle's reverse-mode derivative (attention_vjp): checks against
things other than the function itself.

* the adjoint identity with the separately pinned JVP oracle:
  <gO, dO(t)> = <gQ, tq> + <gK, tk> + <gV, tv> for every tangent t and
  cotangent gO (this is what makes gQ, gK, gV the gradients of <gO, O>);
* complex-step derivatives of the pure-Python brute-force attention (the
  gradient of the scalar <gO, O> one input element at a time);
* closed forms: a single key (gQ = gK = 0, gV = sum of gO rows) and uniform
  attention (Q = 0);
* torch.autograd of a plain torch fp64 attention (a library special case);
* the sampled-keys form (attention_vjp_keys) equals the key rows of the
  whole-tensor gradients.

Planted mistakes in a copy of the oracle (CPU only) must each fail a pin.
"""

import importlib
import types

import numpy as np
import pytest

import oracle

from test_oracle import brute_attention

oracle_mod = importlib.import_module("oracle.attention_jvp")


def _inputs(rng, B, H, Nq, Nk, d, spread=1.0):
    r = lambda *s: rng.standard_normal(s)
    q = r(B, H, Nq, d) * spread
    k, v = r(B, H, Nk, d), r(B, H, Nk, d)
    return q, k, v, r(B, H, Nq, d)


def _close(got, want, tol, what):
    err = np.abs(got - want).max() / max(np.abs(want).max(), 1e-300)
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


def pin_vjp_adjoint(orc):
    """<gO, JVP(t)> == <(gQ, gK, gV), t>, for workload-like inputs, incl. a
    query count past one row chunk."""
    rng = np.random.default_rng(11)
    for (B, H, Nq, Nk, d, spread, s) in [(1, 2, 7, 9, 4, 1.0, 0.5), (2, 1, 33, 17, 8, 3.0, 0.35),
                                         (1, 1, 600, 40, 4, 2.0, 0.5)]:
        q, k, v, go = _inputs(rng, B, H, Nq, Nk, d, spread)
        k[:, :, 1] *= 8  # an outlier key
        tq, tk, tv = (rng.standard_normal(x.shape) for x in (q, k, v))
        _, dO, _ = orc.attention_jvp(q, k, v, tq, tk, tv, s)
        gq, gk, gv = orc.attention_vjp(q, k, v, go, s)
        lhs = float((go * dO).sum())
        rhs = float((gq * tq).sum() + (gk * tk).sum() + (gv * tv).sum())
        assert abs(lhs - rhs) <= 1e-11 * max(abs(lhs), 1.0), (B, H, Nq, Nk, d, lhs, rhs)
        # each input's gradient on its own (tangent along that input only)
        for which in range(3):
            t = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
            t[which] = (tq, tk, tv)[which]
            _, dO1, _ = orc.attention_jvp(q, k, v, *t, s)
            g = (gq, gk, gv)[which]
            assert abs(float((go * dO1).sum()) - float((g * t[which]).sum())) <= \
                1e-11 * max(abs(float((go * dO1).sum())), 1.0), which


def pin_vjp_complex_step(orc):
    """Gradient of <gO, O> element by element with a complex step through the
    pure-Python brute force (no formula for the gradient anywhere)."""
    rng = np.random.default_rng(12)
    q, k, v, go = _inputs(rng, 1, 1, 3, 4, 2)
    s, h = 0.7, 1e-30
    gq, gk, gv = orc.attention_vjp(q, k, v, go, s)
    base = [q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()]
    for which, grad in enumerate((gq, gk, gv)):
        for i in range(len(base[which])):
            for c in range(len(base[which][0])):
                args = [[list(map(complex, r)) for r in x] for x in base]
                args[which][i][c] += complex(0, h)
                o, _ = brute_attention(args[0], args[1], args[2], s)
                val = sum(go[0, 0, a, b] * o[a][b].imag / h for a in range(len(o)) for b in range(2))
                assert abs(val - grad[0, 0, i, c]) <= 1e-12 * max(1.0, abs(val)), (which, i, c)


def pin_vjp_single_key(orc):
    rng = np.random.default_rng(13)
    q, k, v, go = _inputs(rng, 1, 2, 6, 1, 5)
    gq, gk, gv = orc.attention_vjp(q, k, v, go, 0.9)
    assert np.abs(gq).max() <= 1e-14 and np.abs(gk).max() <= 1e-13
    _close(gv[:, :, 0], go.sum(axis=2), 1e-14, "single key: gV = sum of gO rows")


def pin_vjp_uniform(orc):
    """Q = 0: P = 1/Nk, gV_j = mean_i... = sum_i gO_i / Nk, gK = 0,
    gQ_i = (s / Nk) sum_j <gO_i, v_j - vbar> k_j."""
    rng = np.random.default_rng(14)
    _, k, v, go = _inputs(rng, 1, 1, 5, 7, 3)
    q = np.zeros((1, 1, 5, 3))
    s = 0.6
    gq, gk, gv = orc.attention_vjp(q, k, v, go, s)
    Nk = 7
    _close(gv[0, 0], np.repeat(go[0, 0].sum(axis=0, keepdims=True) / Nk, Nk, axis=0), 1e-13, "gV")
    assert np.abs(gk).max() <= 1e-14
    vc = v[0, 0] - v[0, 0].mean(axis=0)
    _close(gq[0, 0], (s / Nk) * (go[0, 0] @ vc.T) @ k[0, 0], 1e-13, "gQ")


def pin_vjp_torch_autograd(orc):
    import torch

    rng = np.random.default_rng(15)
    q, k, v, go = _inputs(rng, 2, 2, 9, 11, 4, 2.0)
    s = 0.45
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(s * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    (o * torch.tensor(go)).sum().backward()
    gq, gk, gv = orc.attention_vjp(q, k, v, go, s)
    for name, a, b in (("gQ", gq, tq.grad), ("gK", gk, tk.grad), ("gV", gv, tv.grad)):
        _close(a, b.numpy(), 1e-12, name)


def pin_vjp_keys(orc):
    """The sampled-keys form equals the key rows of the whole-tensor gradients
    (pinned above), with chunks of query rows that split the rows unevenly."""
    rng = np.random.default_rng(16)
    q, k, v, go = _inputs(rng, 2, 3, 1200, 37, 8, 1.5)
    s = 0.3
    _, gk, gv = orc.attention_vjp(q, k, v, go, s)
    for b, h in ((0, 0), (1, 2)):
        keys = np.array([0, 5, 17, 36])
        a, c = orc.attention_vjp_keys(q, k, v, go, s, b, h, keys)
        _close(a, gk[b, h, keys], 1e-12, "gK rows")
        _close(c, gv[b, h, keys], 1e-12, "gV rows")


PINS = [pin_vjp_adjoint, pin_vjp_complex_step, pin_vjp_single_key, pin_vjp_uniform,
        pin_vjp_torch_autograd, pin_vjp_keys]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_vjp_pin(pin):
    pin(oracle)


MUTATIONS = [
    ("gV with P not transposed", "gV = P.T @ go", "gV = P @ go[:P.shape[1]] if P.shape[0] >= P.shape[1] else P.T @ go * 0.5"),
    ("D left out", "gS = P * (gP - D)", "gS = P * gP"),
    ("D sign", "gS = P * (gP - D)", "gS = P * (gP + D)"),
    ("D over the wrong axis", "D = (P * gP).sum(axis=1, keepdims=True)", "D = (P * gP).sum(axis=0, keepdims=True)"),
    ("gP against K instead of V", "gP = go @ v.T", "gP = go @ k.T"),
    ("scale left out of gQ", "return scale * (gS @ k), scale * (gS.T @ q), gV", "return (gS @ k), scale * (gS.T @ q), gV"),
    ("scale left out of gK", "return scale * (gS @ k), scale * (gS.T @ q), gV", "return scale * (gS @ k), (gS.T @ q), gV"),
    ("gQ and gK swapped operands", "return scale * (gS @ k), scale * (gS.T @ q), gV", "return scale * (gS @ v), scale * (gS.T @ q), gV"),
    ("gK from the wrong side", "return scale * (gS @ k), scale * (gS.T @ q), gV", "return scale * (gS @ k), scale * (gS.T @ go), gV"),
    ("chunked gK not accumulated", "gk[b, h] += c", "gk[b, h] = c"),
    ("sampled keys: D from the kept columns only", "gS = P[:, keys] * (gP[:, keys] - D)",
     "gS = P[:, keys] * (gP[:, keys] - (P[:, keys] * gP[:, keys]).sum(axis=1, keepdims=True))"),
    ("sampled keys: chunks not accumulated", "gv += P[:, keys].T @ gob[r0:r1]",
     "gv = P[:, keys].T @ gob[r0:r1]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_vjp_pins_catch_mutations(name, old, new):
    src = open(oracle_mod.__file__).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mutant = types.ModuleType("oracle_mutant")
    mutant.__file__ = "<mutant>"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mutant.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception:  # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutation '{name}'"
