"""GPU parity of the backward pass (attn_bwd) against the fp64 oracle's
reverse-mode derivative, at reduced sizes in full and at a full video size on
sampled rows plus the adjoint identity with the JVP kernel.

The cotangent gO is drawn like dQ (N(0, 0.1^2), bf16); O and lse come from
the forward kernel.  Gate (the pages state none for gradients): per output,
relative Frobenius error <= 1e-2 and max-abs error <= 2e-2 * max|reference|
(gK and gV sum over all queries, so their size grows with Nq)."""

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle
from workloads import make_inputs

from _gpu import NAMES, metrics, to_device

pytestmark = pytest.mark.gpu


def _gate(label, got, want):
    for name, a, b in zip(("gQ", "gK", "gV"), got, want):
        a = a.double().cpu().numpy() if isinstance(a, torch.Tensor) else a
        m = metrics(a, b)
        print(f"[{label}] {name}: rel-Frobenius {m['rel_frob']:.3e} max-abs/max|ref| "
              f"{m['max_rel']:.3e} max-abs {m['max_abs']:.3e}", flush=True)
        assert np.isfinite(a).all(), (label, name)
        if np.abs(b).max() < 1e-12:  # an exactly zero gradient (one key: gQ = gK = 0)
            assert m["max_abs"] <= 1e-5, (label, name, m)
        else:
            assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2, (label, name, m)


def _run(g, s):
    print(f"  launch attn_bwd q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}", flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    out = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(256, 256), (300, 200), (129, 515), (64, 1000), (1000, 64),
                                   (1, 17), (17, 1), (257, 63)])
def test_backward_reduced(Nq, Nk, d):
    x, s = make_inputs("image_dit", Nq=Nq, Nk=Nk, heads=[0, 1])
    if d == 64:
        x = {n: t[..., :64].contiguous() for n, t in x.items()}
        s = 0.125
    g = to_device(x)
    got = _run(g, s)
    want = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], s)
    _gate(f"bwd {Nq}x{Nk} d={d}", got, want)


@pytest.mark.parametrize("name", ["video_14b", "video_1p3b"])
def test_backward_recipes_reduced(name):
    x, s = make_inputs(name, Nq=700, Nk=900, heads=[0, 1])
    g = to_device(x)
    got = _run(g, s)
    want = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], s)
    _gate(f"bwd {name} 700x900", got, want)


def test_backward_video_full_size():
    """One head of the 1.3B-video shape (N = 32760): gQ on sampled query rows
    and gK, gV (sums over all 32760 queries) on sampled key rows against the
    oracle, and all three through the adjoint identity <gO, dO(t)> = <gQ, tq> +
    <gK, tk> + <gV, tv> with the JVP kernel's dO for independent tangents."""
    x, s = make_inputs("video_1p3b", heads=[0])
    g = to_device(x)
    go = g["dq"]
    gq, gk, gv = _run(g, s)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(32760, 40, replace=False), [0, 32759]]))
    # gQ rows: oracle on the sampled query rows (gQ of a row needs only that row)
    ref = oracle.attention_vjp(x["q"][:, :, rows], x["k"], x["v"], x["dq"][:, :, rows], s)[0]
    m = metrics(gq[0, 0, rows].double().cpu().numpy(), ref[0, 0])
    print(f"[bwd video_1p3b full] gQ rows: {m}", flush=True)
    assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2
    # adjoint identity with independent random tangents
    tg = torch.Generator(device="cpu").manual_seed(5)
    t = {n: (torch.randn(g[n].shape, generator=tg) * 0.1).to(torch.bfloat16).cuda()
         for n in ("q", "k", "v")}
    _, dO, _ = ajvp.attn_jvp_fwd(g["q"], g["k"], g["v"], t["q"], t["k"], t["v"], scale=s)
    torch.cuda.synchronize()
    lhs = float((go.double() * dO.double()).sum())
    rhs = float((gq.double() * t["q"].double()).sum() + (gk.double() * t["k"].double()).sum()
                + (gv.double() * t["v"].double()).sum())
    print(f"[bwd video_1p3b full] adjoint: lhs {lhs:.6e} rhs {rhs:.6e}", flush=True)
    scale_ref = float((go.double().abs() * dO.double().abs()).sum())
    assert abs(lhs - rhs) <= 1e-2 * scale_ref
    assert torch.isfinite(gk).all() and torch.isfinite(gv).all()
    # gK, gV rows element by element: sampled keys (each a sum over all 32760
    # queries) against the oracle, which processes every query row for them
    keys = np.unique(np.concatenate([rng.choice(32760, 40, replace=False), [0, 32759]]))
    rk, rv = oracle.attention_vjp_keys(x["q"], x["k"], x["v"], x["dq"], s, 0, 0, keys)
    for name, got, want in (("gK", gk, rk), ("gV", gv, rv)):
        m = metrics(got[0, 0, keys].double().cpu().numpy(), want)
        print(f"[bwd video_1p3b full] {name} rows: {m}", flush=True)
        assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2, (name, m)


def test_backward_text_cross_full_size():
    """The cross-attention shape (32760 queries x 512 keys, 12 heads) at the
    launch configuration the benchmark times (the gK/gV kernel split over
    query ranges, partial sums added by a second kernel): heads 0 and 11
    against the oracle in full."""
    x, s = make_inputs("text_cross")
    g = to_device(x)
    gq, gk, gv = _run(g, s)
    for h in (0, 11):
        sub = {n: x[n][:, h:h + 1].contiguous() for n in ("q", "k", "v", "dq")}
        want = oracle.attention_vjp(sub["q"], sub["k"], sub["v"], sub["dq"], s)
        _gate(f"bwd text_cross head {h}", (gq[:, h:h + 1], gk[:, h:h + 1], gv[:, h:h + 1]), want)


def test_backward_workspace_and_pool_agree():
    x, s = make_inputs("image_dit", Nq=333, Nk=271, heads=[0, 1, 2])
    g = to_device(x)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    a = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s)
    B, H, Nq, d = g["q"].shape
    ws = torch.empty(ajvp.attn_bwd_workspace_bytes(B, H, Nq, g["k"].shape[2], d),
                     dtype=torch.uint8, device="cuda")
    b = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s, workspace=ws)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
