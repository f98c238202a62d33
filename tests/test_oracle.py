"""Pins for the fp64 oracle: checks against things other than the oracle itself.

The pages about rCM name the computation (attention and its JVP in one pass;
Anthology of the SOTA record LIT-783, "Key takeaways", "JVP at production
scale", paper §3.2 / App. C) but print no worked value, so the oracle is pinned
to mathematics:

* complex-step derivatives of a pure-Python brute-force attention (no NumPy),
  which give the directional derivative to machine precision with no formula
  for it written anywhere;
* central finite differences (eps = 1e-6) on inputs drawn like the workloads'
  (row maxima 5-20, x8 outlier rows);
* exact identities: linearity in the tangent, JVP(0, 0, dV) = attention(Q, K, dV),
  invariance under adding one vector to every key, dlse = d(lse);
* closed forms: uniform attention (Q = 0), a single key, and the hand-derived
  fixtures in tests/golden/closed_forms.json;
* torch.func.jvp of a plain torch fp64 attention (a library special case).

Every pin is a function of an oracle module, so ``test_pins_catch_mutations``
can plant plausible mistakes in a copy of the oracle (on the CPU) and show that
the pins fail on each.
"""

import cmath
import importlib
import json
import math
import os

import numpy as np
import pytest

import oracle

oracle_mod = importlib.import_module("oracle.attention_jvp")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


# ----------------------------------------------------------------------------
# independent brute force: pure Python, works on complex numbers
# ----------------------------------------------------------------------------

def brute_attention(q, k, v, scale):
    """Softmax attention with nested Python loops; q, k, v are lists of rows.

    Accepts complex entries so that a complex step gives the exact derivative.
    The subtracted max uses real parts only (any constant shift is exact).
    """
    outs, lses = [], []
    for qi in q:
        logits = [scale * sum(a * b for a, b in zip(qi, kj)) for kj in k]
        mx = max(s.real for s in logits)
        w = [cmath.exp(s - mx) for s in logits]
        tot = sum(w)
        outs.append([sum(w[j] * v[j][c] for j in range(len(k))) / tot for c in range(len(v[0]))])
        lses.append(mx + cmath.log(tot))
    return outs, lses


def complex_step_jvp(q, k, v, dq, dk, dv, scale, h=1e-30):
    def lift(x, t):
        return [[complex(a, h * b) for a, b in zip(xr, tr)] for xr, tr in zip(x, t)]

    o, lse = brute_attention(lift(q, dq), lift(k, dk), lift(v, dv), scale)
    O = np.array([[z.real for z in r] for r in o])
    dO = np.array([[z.imag / h for z in r] for r in o])
    L = np.array([z.real for z in lse])
    dL = np.array([z.imag / h for z in lse])
    return O, dO, L, dL


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def _inputs(rng, B, H, Nq, Nk, d, tsig=0.1):
    q, k, v = _rand(rng, B, H, Nq, d), _rand(rng, B, H, Nk, d), _rand(rng, B, H, Nk, d)
    dq, dk, dv = (_rand(rng, B, H, n, d, sigma=tsig) for n in (Nq, Nk, Nk))
    return q, k, v, dq, dk, dv


def _close(a, b, rel, what=""):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max()
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:.1e} * {scale:.3e}"


def _workload_like(rng, Nq, Nk, d):
    """Tiny inputs with the workloads' value structure: per-row max logits in
    [5, 20] (the 1.3B video shape) and x8 outlier rows (the 14B video shape)."""
    scale = 1.0 / math.sqrt(d)
    q, k, v, dq, dk, dv = _inputs(rng, 1, 1, Nq, Nk, d)
    t = rng.uniform(5.0, 20.0, size=Nq)
    m = (scale * q[0, 0] @ k[0, 0].T).max(axis=1)
    m = np.where(m > 0.05, m, 0.05)
    q[0, 0] *= (t / m)[:, None]
    for x in (k, v):
        idx = rng.choice(Nk, size=max(1, Nk // 10), replace=False)
        x[0, 0, idx] *= 8.0
    return (q, k, v, dq, dk, dv), scale


# ----------------------------------------------------------------------------
# pins (each takes an oracle module)
# ----------------------------------------------------------------------------

def pin_complex_step(orc):
    rng = np.random.default_rng(1)
    for (Nq, Nk, d, scale) in [(1, 1, 1, 1.0), (3, 5, 2, 0.7), (4, 7, 3, 1.3), (8, 8, 4, 0.5), (5, 2, 4, 2.0)]:
        q, k, v, dq, dk, dv = _inputs(rng, 1, 1, Nq, Nk, d, tsig=1.0)
        O, dO, L, dL = orc.attention_jvp(q, k, v, dq, dk, dv, scale, with_dlse=True)
        cO, cdO, cL, cdL = complex_step_jvp(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                            dq[0, 0].tolist(), dk[0, 0].tolist(), dv[0, 0].tolist(), scale)
        _close(O[0, 0], cO, 1e-12, "O")
        _close(dO[0, 0], cdO, 1e-12, "dO")
        _close(L[0, 0], cL, 1e-12, "lse")
        _close(dL[0, 0], cdL, 1e-11, "dlse")
        fO, fL = orc.attention(q, k, v, scale)
        _close(fO[0, 0], cO, 1e-12, "forward O")
        _close(fL[0, 0], cL, 1e-12, "forward lse")


def pin_finite_difference(orc):
    eps = 1e-6
    rng = np.random.default_rng(2)
    cases = []
    for (Nq, Nk, d) in [(1, 1, 4), (3, 5, 4), (17, 33, 8), (3, 1, 8)]:
        cases.append((_inputs(rng, 1, 2, Nq, Nk, d, tsig=1.0), 1.0 / math.sqrt(d)))
    for (Nq, Nk, d) in [(17, 33, 8), (9, 40, 4)]:
        cases.append(_workload_like(rng, Nq, Nk, d))
    for (q, k, v, dq, dk, dv), scale in cases:
        O, dO, L, dL = orc.attention_jvp(q, k, v, dq, dk, dv, scale, with_dlse=True)
        Op, Lp = orc.attention(q + eps * dq, k + eps * dk, v + eps * dv, scale)
        Om, Lm = orc.attention(q - eps * dq, k - eps * dk, v - eps * dv, scale)
        _close(dO, (Op - Om) / (2 * eps), 1e-6, "dO vs central FD")
        _close(dL, (Lp - Lm) / (2 * eps), 1e-6, "dlse vs central FD")


def pin_linearity(orc):
    rng = np.random.default_rng(3)
    q, k, v, a1, b1, c1 = _inputs(rng, 2, 2, 9, 13, 8)
    a2, b2, c2 = _rand(rng, 2, 2, 9, 8), _rand(rng, 2, 2, 13, 8), _rand(rng, 2, 2, 13, 8)
    s = 0.35
    _, d1, _ = orc.attention_jvp(q, k, v, a1, b1, c1, s)
    _, d2, _ = orc.attention_jvp(q, k, v, a2, b2, c2, s)
    _, d12, _ = orc.attention_jvp(q, k, v, a1 + 2.5 * a2, b1 + 2.5 * b2, c1 + 2.5 * c2, s)
    _close(d12, d1 + 2.5 * d2, 1e-12, "linearity")
    _, dm, _ = orc.attention_jvp(q, k, v, -3.0 * a1, -3.0 * b1, -3.0 * c1, s)
    _close(dm, -3.0 * d1, 1e-12, "homogeneity")


def pin_value_tangent_identity(orc):
    rng = np.random.default_rng(4)
    q, k, v, dq, dk, dv = _inputs(rng, 1, 3, 11, 19, 8)
    z = np.zeros_like
    s = 1.0 / math.sqrt(8)
    _, dO, _ = orc.attention_jvp(q, k, v, z(dq), z(dk), dv, s)
    ref, _ = orc.attention(q, k, dv, s)
    _close(dO, ref, 1e-13, "JVP(0,0,dV) = attention(Q,K,dV)")
    # and the same with the brute force on one head
    bo, _ = brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), dv[0, 0].tolist(), s)
    _close(dO[0, 0], np.array([[z_.real for z_ in r] for r in bo]), 1e-13, "vs brute force")


def pin_key_shift_invariance(orc):
    rng = np.random.default_rng(5)
    q, k, v, _, _, _ = _inputs(rng, 1, 2, 7, 23, 8)
    c = rng.standard_normal(8)
    dk = np.broadcast_to(c, k.shape).copy()
    z = np.zeros_like
    _, dO, _, dL = orc.attention_jvp(q, k, v, z(q), dk, z(v), 0.4, with_dlse=True)
    bound = 1e-13 * np.linalg.norm(c) * np.abs(v).max() * np.abs(q).max() * 8
    assert np.abs(dO).max() <= bound, np.abs(dO).max()
    # lse does move: its tangent is s * q_i . c for every key.
    _close(dL, 0.4 * (q @ c), 1e-12, "dlse under a common key shift")


def pin_uniform_closed_form(orc):
    """Q = 0: P = 1/Nk, O = mean v, lse = ln Nk, dO_i = s dq_i^T Cov(K, V) + mean dv."""
    rng = np.random.default_rng(6)
    Nq, Nk, d, s = 5, 9, 6, 0.8
    _, k, v, dq, dk, dv = _inputs(rng, 1, 1, Nq, Nk, d, tsig=1.0)
    q = np.zeros((1, 1, Nq, d))
    O, dO, L = orc.attention_jvp(q, k, v, dq, dk, dv, s)
    K, V = k[0, 0], v[0, 0]
    cov = (K - K.mean(0)).T @ (V - V.mean(0)) / Nk
    _close(O[0, 0], np.broadcast_to(V.mean(0), (Nq, d)), 1e-13, "uniform O")
    _close(L[0, 0], np.full(Nq, math.log(Nk)), 1e-13, "uniform lse")
    _close(dO[0, 0], s * dq[0, 0] @ cov + dv[0, 0].mean(0), 1e-12, "uniform dO")


def pin_single_key(orc):
    rng = np.random.default_rng(7)
    q, k, v, dq, dk, dv = _inputs(rng, 2, 2, 6, 1, 8, tsig=1.0)
    O, dO, L, dL = orc.attention_jvp(q, k, v, dq, dk, dv, 0.3, with_dlse=True)
    _close(O, np.broadcast_to(v, O.shape), 1e-14, "one key: O = v0")
    _close(dO, np.broadcast_to(dv, dO.shape), 1e-14, "one key: dO = dv0")
    _close(L, 0.3 * (q @ k.swapaxes(-1, -2))[..., 0], 1e-14, "one key: lse = s q.k0")
    _close(dL, 0.3 * ((dq @ k.swapaxes(-1, -2)) + (q @ dk.swapaxes(-1, -2)))[..., 0], 1e-13,
           "one key: dlse = s(dq.k0 + q.dk0)")


def pin_torch_func_jvp(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    q, k, v, dq, dk, dv = _inputs(rng, 2, 3, 10, 14, 8)
    s = 1.0 / math.sqrt(8)

    def f(q_, k_, v_):
        a = torch.softmax(s * (q_ @ k_.transpose(-1, -2)), dim=-1)
        return a @ v_, torch.logsumexp(s * (q_ @ k_.transpose(-1, -2)), dim=-1)

    T = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    (tO, tL), (tdO, tdL) = torch.func.jvp(f, (T(q), T(k), T(v)), (T(dq), T(dk), T(dv)))
    O, dO, L, dL = orc.attention_jvp(q, k, v, dq, dk, dv, s, with_dlse=True)
    _close(O, tO.numpy(), 1e-12, "O vs torch")
    _close(dO, tdO.numpy(), 1e-12, "dO vs torch.func.jvp")
    _close(L, tL.numpy(), 1e-12, "lse vs torch")
    _close(dL, tdL.numpy(), 1e-12, "dlse vs torch.func.jvp")


def pin_golden(orc):
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        arr = lambda key: np.array(case[key], dtype=np.float64)[None, None]
        O, dO, L, dL = orc.attention_jvp(arr("q"), arr("k"), arr("v"), arr("dq"), arr("dk"), arr("dv"),
                                         case["scale"], with_dlse=True)
        for name, got in (("O", O), ("dO", dO), ("lse", L), ("dlse", dL)):
            want = np.array(case[name], dtype=np.float64)
            assert np.allclose(got[0, 0], want, rtol=1e-14, atol=1e-14), (case["name"], name, got, want)


def pin_rows_match_whole(orc):
    rng = np.random.default_rng(9)
    q, k, v, dq, dk, dv = _inputs(rng, 2, 2, 40, 21, 8)
    O, dO, L = orc.attention_jvp(q, k, v, dq, dk, dv, 0.5)
    rows = np.array([39, 0, 17, 17, 5])
    o, do, l_ = orc.attention_jvp_rows(q, k, v, dq, dk, dv, 0.5, 1, 0, rows)
    assert np.array_equal(o, O[1, 0, rows]) and np.array_equal(do, dO[1, 0, rows])
    assert np.array_equal(l_, L[1, 0, rows])


PINS = [pin_complex_step, pin_finite_difference, pin_linearity, pin_value_tangent_identity,
        pin_key_shift_invariance, pin_uniform_closed_form, pin_single_key, pin_torch_func_jvp,
        pin_golden, pin_rows_match_whole]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


def test_brute_force_matches_closed_form():
    """The brute force itself, on the hand-derived fixtures (no oracle involved)."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        O, dO, L, dL = complex_step_jvp(case["q"], case["k"], case["v"], case["dq"], case["dk"],
                                        case["dv"], case["scale"])
        assert np.allclose(O, case["O"], rtol=1e-14, atol=1e-14), case["name"]
        assert np.allclose(dO, case["dO"], rtol=1e-13, atol=1e-13), case["name"]
        assert np.allclose(L, case["lse"], rtol=1e-14, atol=1e-14), case["name"]
        assert np.allclose(dL, case["dlse"], rtol=1e-13, atol=1e-13), case["name"]


# ----------------------------------------------------------------------------
# planted mistakes (CPU only): each plausible slip in the oracle must fail a pin
# ----------------------------------------------------------------------------

MUTATIONS = [
    ("dropped P dV term", "dO = dP @ v + P @ dv", "dO = dP @ v"),
    ("dropped dP V term", "dO = dP @ v + P @ dv", "dO = P @ dv"),
    ("wrong sign of mu", "dP = P * (dS - mu[:, None])", "dP = P * (dS + mu[:, None])"),
    ("mu not subtracted", "dP = P * (dS - mu[:, None])", "dP = P * dS"),
    ("scale missing from dS", "dS = scale * (dq @ k.T + q @ dk.T)", "dS = (dq @ k.T + q @ dk.T)"),
    ("dropped Q dK term", "dS = scale * (dq @ k.T + q @ dk.T)", "dS = scale * (dq @ k.T)"),
    ("dropped dQ K term", "dS = scale * (dq @ k.T + q @ dk.T)", "dS = scale * (q @ dk.T)"),
    ("wrong operand in dS", "dS = scale * (dq @ k.T + q @ dk.T)", "dS = scale * (dq @ k.T + dq @ dk.T)"),
    ("mu over the wrong axis", "mu = (P * dS).sum(axis=1)", "mu = (P * dS).sum(axis=1) / P.shape[1]"),
    ("log2 instead of ln", "lse = m[:, 0] + np.log(l[:, 0])", "lse = m[:, 0] + np.log2(l[:, 0])"),
    ("max left out of lse", "lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])"),
    ("unnormalised P", "P = E / l", "P = E / l.max()"),
    ("scale missing from S", "S = scale * (q @ k.T)", "S = (q @ k.T)"),
    ("keys and values swapped", "O = P @ v", "O = P @ k"),
    ("dlse wrong", "return O, dO, lse, mu", "return O, dO, lse, mu * scale"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutations(name, old, new):
    src = open(oracle_mod.__file__).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mutant_src = src.replace(old, new)
    import types

    mutant = types.ModuleType("oracle_mutant")
    mutant.__file__ = "<mutant>"
    exec(compile(mutant_src, "<mutant>", "exec"), mutant.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception:  # noqa: BLE001 - any failure (assert or shape error) counts
            failed.append(pin.__name__)
    assert failed, f"no pin caught the mutation '{name}'"
