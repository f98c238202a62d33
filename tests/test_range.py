"""Inputs far outside fp16's range through the bf16 paths (GPU).

The second contraction (P and s P dS against V and dV) runs on fp16 operands,
which hold magnitudes from 2^-24 to 65504 only, while bf16 inputs span
2^-133 .. 3.4e38.  The library scales V and dV by per-slice powers of two
and s P dS by a per-wave power of two chosen from a bound of |s dS|, and
undoes both exactly in fp32.  Three kinds of check:

* power-of-two equivariance, bit for bit: multiplying (V, dV) by 2^k
  multiplies O, dO by 2^k exactly; multiplying every tangent by 2^k
  multiplies dO and the tangent of lse by 2^k and leaves O, lse unchanged
  (every product and sum moves by whole binades);
* parity with the fp64 oracle for values that overflow or underflow fp16
  (|V|, |dV| up to ~1e6, |s dS| ~ 1e4, magnitudes ~1e-6..1e-9), on the
  256-row kernel, the short-key kernel, frozen keys, split-KV and the
  forward pass alone.  The gate is the bf16 gate made scale-free: relative
  Frobenius error <= 1e-2 and max-abs error <= 5e-3 of the largest reference
  magnitude (2e-2 against |O| ~ 4 for the unit-scale recipes);
* NaN and Inf inputs propagate: an output element is non-finite exactly
  where the oracle's is, and the finite ones pass the gate.
"""

import math

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle

from _gpu import metrics

pytestmark = pytest.mark.gpu

S128 = 1.0 / math.sqrt(128)
REL_FROB = 1e-2
MAX_REL = 5e-3


def _rand(H, Nq, Nk, seed, sig=(1.0, 1.0, 1.0, 0.1, 0.1, 0.1), d=128):
    g = torch.Generator().manual_seed(seed)
    n = {"q": Nq, "k": Nk, "v": Nk, "dq": Nq, "dk": Nk, "dv": Nk}
    return {name: (torch.randn(1, H, n[name], d, generator=g) * sg).to(torch.bfloat16)
            for name, sg in zip(("q", "k", "v", "dq", "dk", "dv"), sig)}


def _pow2(t, k):
    """t * 2^k, exact in bf16 while the values stay normal."""
    return (t.float() * 2.0 ** k).to(torch.bfloat16)


def _jvp_ex(x, scale=S128, frozen=False, out_dtype=torch.float32):
    g = {n: t.cuda() for n, t in x.items()}
    print(f"  launch jvp_ex q{tuple(g['q'].shape)} k{tuple(g['k'].shape)} frozen={frozen}",
          flush=True)
    out = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], None if frozen else g["dk"],
                               None if frozen else g["dv"], scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in out]


def _oracle(x, scale=S128, frozen=False, with_dlse=False):
    dk = torch.zeros_like(x["dk"]) if frozen else x["dk"]
    dv = torch.zeros_like(x["dv"]) if frozen else x["dv"]
    with np.errstate(all="ignore"):
        return oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], dk, dv, scale,
                                    with_dlse=with_dlse)


def _gate(label, got, want):
    got = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    m = metrics(got, want)
    print(f"[{label}] max-abs {m['max_abs']:.3e} max-abs/max|ref| {m['max_rel']:.3e} "
          f"rel-Frobenius {m['rel_frob']:.3e} max|ref| {np.abs(want).max():.3e}", flush=True)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    assert m["rel_frob"] <= REL_FROB and m["max_rel"] <= MAX_REL, (label, m)


# ---- bit-exact equivariance --------------------------------------------------

@pytest.mark.parametrize("Nk", [300, 1500], ids=["short_kernel", "256row_kernel"])
def test_value_scaling_is_exact(Nk):
    """(V, dV) -> 2^k (V, dV) gives 2^k O and 2^k dO bit for bit, lse and the
    tangent of lse unchanged, for k from -100 to 100 (|V| from ~1e-30 to ~1e30)."""
    x = _rand(2, 300, Nk, seed=Nk)
    o, to, lse, tlse = _jvp_ex(x)
    for k in (20, -30, 100, -100):
        y = dict(x, v=_pow2(x["v"], k), dv=_pow2(x["dv"], k))
        o2, to2, lse2, tlse2 = _jvp_ex(y)
        f = 2.0 ** k
        assert torch.equal(o2, o * f), k
        assert torch.equal(to2, to * f), k
        assert torch.equal(lse2, lse), k
        assert torch.equal(tlse2, tlse), k


@pytest.mark.parametrize("Nk", [300, 1500], ids=["short_kernel", "256row_kernel"])
@pytest.mark.parametrize("frozen", [False, True], ids=["full", "frozen_keys"])
def test_tangent_scaling_is_exact(Nk, frozen):
    """(dQ, dK, dV) -> 2^k (dQ, dK, dV) gives 2^k dO and 2^k mu bit for bit and
    the same O and lse, for k from -40 to 60 (|dS| from ~1e-13 to ~1e17)."""
    x = _rand(2, 300, Nk, seed=7 + Nk)
    o, to, lse, tlse = _jvp_ex(x, frozen=frozen)
    for k in (12, -40, 60):
        y = dict(x, dq=_pow2(x["dq"], k), dk=_pow2(x["dk"], k), dv=_pow2(x["dv"], k))
        o2, to2, lse2, tlse2 = _jvp_ex(y, frozen=frozen)
        f = 2.0 ** k
        assert torch.equal(o2, o), k
        assert torch.equal(lse2, lse), k
        assert torch.equal(to2, to * f), k
        assert torch.equal(tlse2, tlse * f), k


# ---- parity with the oracle outside fp16's range -------------------------------

CASES = {
    # name: sigmas of (q, k, v, dq, dk, dv)
    "V_dV_1e6": (1.0, 1.0, 2e5, 0.1, 0.1, 2e4),
    "sdS_1e4": (1.0, 1.0, 1.0, 2.5e3, 2.5e3, 0.1),
    "sdS_1e4_dV_0": (1.0, 1.0, 1.0, 2.5e3, 2.5e3, 0.0),
    "tiny_all": (1.0, 1.0, 1e-6, 1e-8, 1e-8, 1e-7),
    "V_tiny_tangents_huge": (1.0, 1.0, 1e-5, 1e3, 1e3, 1e-3),
    "V_huge_dV_tiny": (1.0, 1.0, 1e5, 0.1, 0.1, 1e-6),
    # s dS far below what dV's exponent leaves it (mu from its own exponent)
    "dV_huge_dS_tiny": (1.0, 1.0, 1e-6, 1e-4, 1e-4, 1e5),
    # row norms whose fp32 sums of squares underflow or overflow (the exact
    # fp64 sums take over)
    "dQ_tiny_dK_huge": (1.0, 1.0, 1.0, 1e-20, 1e12, 0.1),
    "dQ_huge_dK_tiny": (1.0, 1.0, 1.0, 1e18, 1e-3, 0.1),
}


@pytest.mark.parametrize("Nk", [300, 1500], ids=["short_kernel", "256row_kernel"])
@pytest.mark.parametrize("case", list(CASES))
def test_out_of_fp16_range_vs_oracle(case, Nk):
    x = _rand(2, 300, Nk, seed=list(CASES).index(case), sig=CASES[case])
    ref = _oracle(x, with_dlse=True)
    sds = S128 * (x["dq"].double() @ x["k"].double().transpose(-1, -2)
                  + x["q"].double() @ x["dk"].double().transpose(-1, -2))
    print(f"  {case}: max|V| {x['v'].float().abs().max():.3e} max|dV| "
          f"{x['dv'].float().abs().max():.3e} max|s dS| {sds.abs().max():.3e}", flush=True)
    for out_dtype in (torch.float32, torch.bfloat16):
        o, to, lse, tlse = _jvp_ex(x, out_dtype=out_dtype)
        tag = f"{case} Nk={Nk} {str(out_dtype)[6:]}"
        _gate(tag + " O", o, ref[0])
        _gate(tag + " dO", to, ref[1])
        _gate(tag + " lse", lse, ref[2])
        _gate(tag + " tlse", tlse, ref[3])


@pytest.mark.parametrize("case", ["sdS_1e4", "tiny_all", "V_dV_1e6"])
def test_out_of_fp16_range_frozen_splitkv_forward(case):
    """The frozen-key kernel (dK = dV = NULL), split-KV with its merge, and the
    forward pass alone, on the same ranges."""
    x = _rand(2, 200, 1100, seed=3, sig=CASES[case])
    g = {n: t.cuda() for n, t in x.items()}
    fz = _oracle(x, frozen=True)
    print(f"  launch frozen/splitkv/fwd {case}", flush=True)
    o, to, lse, _ = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], None, None, scale=S128)
    torch.cuda.synchronize()
    _gate(f"{case} frozen O", o.cpu(), fz[0])
    _gate(f"{case} frozen dO", to.cpu(), fz[1])
    full = _oracle(x)
    for ns in (3, 0):
        o, to, lse, _ = ajvp.attn_jvp_fwd_splitkv(g["q"], g["k"], g["v"], g["dq"], g["dk"],
                                                  g["dv"], scale=S128, nsplit=ns)
        torch.cuda.synchronize()
        _gate(f"{case} splitkv {ns} O", o.cpu(), full[0])
        _gate(f"{case} splitkv {ns} dO", to.cpu(), full[1])
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=S128)
    torch.cuda.synchronize()
    _gate(f"{case} forward O", o.cpu(), full[0])
    _gate(f"{case} forward lse", lse.cpu(), full[2])
    o, lse = ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=S128, nsplit=4)
    torch.cuda.synchronize()
    _gate(f"{case} forward splitkv O", o.cpu(), full[0])


def test_forward_value_scaling_is_exact():
    x = _rand(2, 600, 1300, seed=11)
    g = {n: t.cuda() for n, t in x.items()}
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=S128)
    for k in (24, -60):
        o2, lse2 = ajvp.attn_fwd(g["q"], g["k"], _pow2(x["v"], k).cuda(), scale=S128)
        torch.cuda.synchronize()
        assert torch.equal(o2, o * 2.0 ** k) and torch.equal(lse2, lse), k


# ---- NaN and Inf ------------------------------------------------------------------

@pytest.mark.parametrize("Nk", [200, 1100], ids=["short_kernel", "256row_kernel"])
@pytest.mark.parametrize("value", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_nonfinite_inputs_propagate(value, Nk):
    """One NaN or +Inf in one input: the outputs are non-finite exactly where
    the oracle's are (a row for q, dq; a column for v, dv; everything for k,
    dk), and the rest still matches the oracle."""
    base = _rand(1, 130, Nk, seed=21)
    for name in ("q", "k", "v", "dq", "dk", "dv"):
        x = {n: t.clone() for n, t in base.items()}
        n = x[name].shape[2]
        x[name][0, 0, n // 3, 5] = value
        got = _jvp_ex(x)
        ref = _oracle(x)
        for oname, gt, rf in zip(("O", "dO", "lse"), got[:3], ref):
            gt = gt.double().numpy()
            bad_g, bad_r = ~np.isfinite(gt), ~np.isfinite(rf)
            print(f"  {name}={value} {oname}: {bad_g.sum()} non-finite (oracle {bad_r.sum()})",
                  flush=True)
            assert (bad_g == bad_r).all(), (name, oname)
            if (~bad_r).any():
                m = metrics(gt[~bad_r], rf[~bad_r])
                assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (name, oname, m)


# ---- the backward pass ------------------------------------------------------------
# Its fp16 operands are Q^T, gO^T and K^T (per-slice powers of two from their
# largest magnitudes), P (<= 1) and the softmax gradient gS (a per-wave power of
# two from |gS_ij| <= |gO_i| |v_j| + |D_i|).  Gate as tests/test_backward.py:
# relative Frobenius error <= 1e-2, max-abs <= 2e-2 of the largest reference
# magnitude.

def _bwd(x, scale=S128):
    g = {n: t.cuda() for n, t in x.items()}
    print(f"  launch attn_fwd + attn_bwd q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}",
          flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=scale)
    out = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=scale)
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


def _bwd_gate(label, got, want):
    for name, a, b in zip(("gQ", "gK", "gV"), got, want):
        a = a.double().numpy()
        m = metrics(a, b)
        print(f"[{label}] {name}: rel-Frobenius {m['rel_frob']:.3e} max-abs/max|ref| "
              f"{m['max_rel']:.3e} max|ref| {np.abs(b).max():.3e}", flush=True)
        assert np.isfinite(a).all(), (label, name)
        assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2, (label, name, m)


@pytest.mark.parametrize("Nk", [200, 700])
def test_backward_scaling_is_exact(Nk):
    """gO -> 2^k gO gives 2^k (gQ, gK, gV); V -> 2^k V (O with it) gives
    2^k (gQ, gK) and the same gV (gS = P (gO V^T - <gO, O>) is linear in V,
    gV = P^T gO does not involve it), bit for bit.  The cotangent gO is the
    dq draw."""
    x = _rand(2, 300, Nk, seed=31 + Nk)
    base = _bwd(x)
    for k in (24, -30):
        y = dict(x, dq=_pow2(x["dq"], k))
        got = _bwd(y)
        for a, b in zip(got, base):
            assert torch.equal(a, b * 2.0 ** k), k
        y = dict(x, v=_pow2(x["v"], k))
        gq, gk, gv = _bwd(y)
        assert torch.equal(gq, base[0] * 2.0 ** k), k
        assert torch.equal(gk, base[1] * 2.0 ** k), k
        assert torch.equal(gv, base[2]), k


BWD_CASES = {
    # sigmas of (q, k, v, gO = dq); dk, dv unused
    "V_1e6": (1.0, 1.0, 2e5, 0.1),
    "gO_1e5": (1.0, 1.0, 1.0, 2e4),
    "Q_1e5_K_1e-5": (2e4, 2e-5, 1.0, 0.1),
    "K_1e5_Q_1e-5": (2e-5, 2e4, 1.0, 0.1),
    "tiny_V_gO": (1.0, 1.0, 1e-6, 1e-7),
}


@pytest.mark.parametrize("case", list(BWD_CASES))
def test_backward_out_of_fp16_range_vs_oracle(case):
    sq, sk, sv, sg = BWD_CASES[case]
    x = _rand(2, 300, 700, seed=list(BWD_CASES).index(case), sig=(sq, sk, sv, sg, 0.1, 0.1))
    want = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], S128)
    _bwd_gate(f"bwd {case}", _bwd(x), want)


def test_backward_nonfinite_inputs_propagate():
    """A NaN in gO row i or in V: the gradients are non-finite exactly where
    the oracle's are."""
    base = _rand(1, 130, 200, seed=41)
    for name in ("dq", "v", "q"):
        x = {n: t.clone() for n, t in base.items()}
        x[name][0, 0, 17, 5] = float("nan")
        got = _bwd(x)
        with np.errstate(all="ignore"):
            want = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], S128)
        for gname, a, b in zip(("gQ", "gK", "gV"), got, want):
            a = a.double().numpy()
            bad_a, bad_b = ~np.isfinite(a), ~np.isfinite(b)
            print(f"  NaN in {name}: {gname} {bad_a.sum()} non-finite (oracle {bad_b.sum()})",
                  flush=True)
            assert (bad_a == bad_b).all(), (name, gname)
