"""GPU tests of the extended entry points: zero (NULL) tangents and the
frozen-key kernel, the tangent of lse, bf16 outputs, forward attention alone,
and the merge of results over key subsets.

Where the new path must agree bit for bit with the full JVP path (which the
parity tests gate against the oracle), that is checked; every path is also
held to the oracle gate itself."""

import itertools

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle
from workloads import make_inputs

from _gpu import NAMES, check, metrics, to_device

pytestmark = pytest.mark.gpu


def _inputs(name="image_dit", Nq=333, Nk=271, heads=(0, 1, 2)):
    x, s = make_inputs(name, Nq=Nq, Nk=Nk, heads=list(heads))
    return x, to_device(x), s


def _full(g, s, **kw):
    print(f"  launch attn_jvp_fwd_ex q{tuple(g['q'].shape)} k{tuple(g['k'].shape)} {kw}", flush=True)
    out = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"], scale=s, **kw)
    torch.cuda.synchronize()
    return out


def test_ex_equals_classic_entry_point_and_exports_dlse():
    """attn_jvp_fwd_ex with every tangent == attn_jvp_fwd bit for bit; its tlse
    is the tangent of lse (the oracle's mu)."""
    x, g, s = _inputs()
    ref = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)
    o, to, lse, tlse = _full(g, s)
    for a, b in zip(ref, (o, to, lse)):
        assert torch.equal(a, b)
    O, dO, L, dL = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s,
                                        with_dlse=True)
    check("ex image_dit", (o, to, lse), (O, dO, L), fp32=False)
    m = metrics(tlse.double().cpu().numpy(), dL)
    print(f"[ex image_dit] dlse: {m}", flush=True)
    assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2


@pytest.mark.parametrize("d", [64, 128])
def test_null_tangents_equal_zero_tangents(d):
    """Each subset of NULL tangents gives exactly the result of explicit zero
    tensors (for tk = tv = NULL through the frozen-key kernel), within the gate."""
    x, s = make_inputs("image_dit", Nq=200, Nk=300, heads=[0, 1])
    if d == 64:
        x = {n: t[..., :64].contiguous() for n, t in x.items()}
        s = 0.125
    g = to_device(x)
    for mask in range(1, 8):
        drop = [n for i, n in enumerate(("dq", "dk", "dv")) if mask >> i & 1]
        gz = dict(g)
        xz = dict(x)
        for n in drop:
            gz[n] = torch.zeros_like(g[n])
            xz[n] = torch.zeros_like(x[n])
        ref = _full(gz, s)
        kw = {("t" + n[1]): (None if n in drop else g[n]) for n in ("dq", "dk", "dv")}
        print(f"  launch NULL {drop} d={d}", flush=True)
        got = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], scale=s, **kw)
        torch.cuda.synchronize()
        for a, b, name in zip(ref, got, ("O", "dO", "lse", "dlse")):
            assert torch.equal(a, b), (drop, name)
        O, dO, L, dL = oracle.attention_jvp(xz["q"], xz["k"], xz["v"], xz["dq"], xz["dk"], xz["dv"],
                                            s, with_dlse=True)
        check(f"NULL {drop} d={d}", got[:3], (O, dO, L), fp32=False)


def test_frozen_keys_full_size():
    """The text-conditioned cross-attention shape with frozen text keys through
    the frozen-key kernel, on sampled rows of every head (Nq = 32760, Nk = 512)."""
    x, s = make_inputs("text_cross_frozen")
    g = to_device(x)
    print("  launch frozen text_cross_frozen full size", flush=True)
    o, to, lse, tlse = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], None, None, scale=s)
    ref = _full(g, s)  # explicit zero dK, dV through the full kernel
    for a, b in zip(ref, (o, to, lse, tlse)):
        assert torch.equal(a, b)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.choice(32760, 40, replace=False), [0, 32759]]))
    for h in range(x["q"].shape[1]):
        O, dO, L = oracle.attention_jvp_rows(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s,
                                             0, h, rows)
        check(f"frozen h={h}", (o[0, h, rows].cpu(), to[0, h, rows].cpu(), lse[0, h, rows].cpu()),
              (O, dO, L), fp32=False)


def test_bf16_outputs_are_rounded_fp32_outputs():
    x, g, s = _inputs()
    o, to, lse, tlse = _full(g, s)
    ob, tob, lseb, tlseb = _full(g, s, out_dtype=torch.bfloat16)
    assert ob.dtype == torch.bfloat16 and tob.dtype == torch.bfloat16
    assert torch.equal(ob, o.to(torch.bfloat16)) and torch.equal(tob, to.to(torch.bfloat16))
    assert torch.equal(lse, lseb) and torch.equal(tlse, tlseb)
    # frozen kernel, bf16 outputs
    a = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], scale=s)
    b = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], scale=s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(b[0], a[0].to(torch.bfloat16)) and torch.equal(b[1], a[1].to(torch.bfloat16))


@pytest.mark.parametrize("name,Nq,Nk,d", [("image_dit", 333, 271, 128), ("image_dit", 65, 1000, 128),
                                          ("image_dit", 129, 17, 64), ("video_14b", 300, 700, 128)])
def test_forward_only(name, Nq, Nk, d):
    """attn_fwd's O and lse equal the JVP kernel's bit for bit and pass the gate
    against the oracle's forward attention (fp32 and bf16 outputs)."""
    x, s = make_inputs(name, Nq=Nq, Nk=Nk, heads=[0, 1])
    if d == 64:
        x = {n: t[..., :64].contiguous() for n, t in x.items()}
        s = 0.125
    g = to_device(x)
    print(f"  launch attn_fwd {name} Nq={Nq} Nk={Nk} d={d}", flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    ob, lseb = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s, out_dtype=torch.bfloat16)
    ref = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[2])
    assert torch.equal(ob, o.to(torch.bfloat16)) and torch.equal(lseb, lse)
    O, L = oracle.attention(x["q"], x["k"], x["v"], s)
    check(f"fwd {name} {Nq}x{Nk} d={d}", (o, None, lse), (O, None, L), fp32=False)


@pytest.mark.parametrize("name", ["video_1p3b", "video_14b", "text_cross", "image_dit"])
def test_forward_only_full_size(name):
    """attn_fwd at the full workload sizes (the launch configuration the
    forward benchmark times: 512-row workgroups, two row blocks per wave)
    returns the JVP kernel's O and lse bit for bit; the JVP kernel itself is
    held to the oracle at these sizes by the parity tests."""
    x, s = make_inputs(name)
    g = to_device(x)
    print(f"  launch attn_fwd / attn_jvp_fwd {name} q{tuple(g['q'].shape)}", flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    ref = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[2])
    # and a few rows against the oracle directly
    rows = [0, 1, x["q"].shape[2] // 2, x["q"].shape[2] - 1]
    O, L = oracle.attention(x["q"][:, :, rows], x["k"], x["v"], s)
    check(f"fwd {name} full, rows {rows}", (o[:, :, rows], None, lse[:, :, rows]), (O, None, L),
          fp32=False)


@pytest.mark.parametrize("parts", [2, 5])
def test_merge_of_key_splits(parts):
    """Results over disjoint key ranges, merged on the GPU, pass the gate
    against the oracle over all keys (JVP and forward-only)."""
    x, s = make_inputs("image_dit", Nq=250, Nk=1000, heads=[0, 1])
    g = to_device(x)
    bounds = np.linspace(0, 1000, parts + 1).astype(int)
    res, fres = [], []
    for j0, j1 in zip(bounds[:-1], bounds[1:]):
        sl = {n: (t if n in ("q", "dq") else t[:, :, j0:j1].contiguous()) for n, t in g.items()}
        print(f"  launch key part {j0}:{j1}", flush=True)
        res.append(ajvp.attn_jvp_fwd_ex(sl["q"], sl["k"], sl["v"], sl["dq"], sl["dk"], sl["dv"], scale=s))
        fres.append(ajvp.attn_fwd(sl["q"], sl["k"], sl["v"], scale=s))
    st = lambda i, rr: torch.stack([r[i] for r in rr]).contiguous()
    lse, o, to, tlse = ajvp.attn_jvp_merge(st(2, res), st(0, res), st(1, res), st(3, res))
    flse, fo, fto, ftlse = ajvp.attn_jvp_merge(st(1, fres), st(0, fres))
    torch.cuda.synchronize()
    assert fto is None and ftlse is None
    O, dO, L, dL = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s,
                                        with_dlse=True)
    check(f"merge {parts}", (o, to, lse), (O, dO, L), fp32=False)
    check(f"merge fwd {parts}", (fo, None, flse), (O, None, L), fp32=False)
    m = metrics(tlse.double().cpu().numpy(), dL)
    assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, m
    # one part: the merge is the identity up to the exp/log round trip of lse
    one = ajvp.attn_jvp_merge(res[0][2][None].contiguous(), res[0][0][None].contiguous(),
                              res[0][1][None].contiguous(), res[0][3][None].contiguous())
    torch.cuda.synchronize()
    assert torch.allclose(one[1], res[0][0], rtol=1e-6, atol=1e-6)
    assert torch.allclose(one[2], res[0][1], rtol=1e-5, atol=1e-5)
