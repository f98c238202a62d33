"""GPU parity over a seeded sweep of call configurations.

Forty configurations drawn once from a fixed seed: batch and head counts,
query and key lengths (biased to the places where the kernels change shape:
multiples of 64 and 128 and one past them, the 16-tile switch between the
128-row and 256-row kernels at 1024 keys), d = 64 or 128, a scale of either
sign, NULL tangents, bf16 outputs, with and without lse and its tangent, and
split-KV ranges.  Every output element is compared with the fp64 oracle
(oracle.attention_jvp on the same bf16 inputs) under the gate of
tests/test_parity.py: max-abs <= 2e-2 and relative Frobenius <= 1e-2.
"""

import math
import random

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle

from _gpu import metrics

pytestmark = pytest.mark.gpu

EDGES_Q = [1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 383, 511, 512, 513]
EDGES_K = [1, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024, 1025, 1088, 1089]


def _configs(n=40, seed=20261203):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        d = rng.choice([64, 128])
        Nq = rng.choice(EDGES_Q) if rng.random() < 0.6 else rng.randint(1, 600)
        Nk = rng.choice(EDGES_K) if rng.random() < 0.6 else rng.randint(1, 1300)
        scale = rng.choice([1.0, -1.0, rng.uniform(-2.5, 2.5)]) / math.sqrt(d)
        out.append(dict(
            i=i, B=rng.choice([1, 2]), H=rng.choice([1, 2, 3]), Nq=Nq, Nk=Nk, d=d, scale=scale,
            null=rng.choice([(), ("dk", "dv"), ("dq",), ("dv",), ("dk",)]),
            bf16_out=rng.random() < 0.25, lse=rng.random() < 0.8, tlse=rng.random() < 0.6,
            nsplit=rng.choice([None, None, None, 0, 2, 3]), tsig=rng.choice([0.1, 1.0])))
    return out


CONFIGS = _configs()


def _inputs(c):
    g = torch.Generator().manual_seed(1000 + c["i"])
    shape = lambda n: (c["B"], c["H"], n, c["d"])
    x = {}
    for name, n, sg in (("q", c["Nq"], 1.0), ("k", c["Nk"], 1.0), ("v", c["Nk"], 1.0),
                        ("dq", c["Nq"], c["tsig"]), ("dk", c["Nk"], c["tsig"]),
                        ("dv", c["Nk"], c["tsig"])):
        x[name] = (torch.randn(*shape(n), generator=g) * sg).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("c", CONFIGS, ids=lambda c: (
    f"{c['i']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_sweep_vs_oracle(c):
    x = _inputs(c)
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    tan = {n: (None if n in c["null"] else g[n]) for n in ("dq", "dk", "dv")}
    print(f"  launch sweep {c}", flush=True)
    if c["nsplit"] is None:
        o, to, lse, tlse = ajvp.attn_jvp_fwd_ex(
            g["q"], g["k"], g["v"], tan["dq"], tan["dk"], tan["dv"], scale=c["scale"],
            lse=c["lse"], tlse=c["tlse"],
            out_dtype=torch.bfloat16 if c["bf16_out"] else torch.float32)
    else:
        o, to, lse, tlse = ajvp.attn_jvp_fwd_splitkv(
            g["q"], g["k"], g["v"], tan["dq"], tan["dk"], tan["dv"], scale=c["scale"],
            nsplit=c["nsplit"], lse=c["lse"], tlse=c["tlse"])
    torch.cuda.synchronize()
    # the oracle takes the zero tensors the NULL tangents stand for
    xz = {n: (torch.zeros_like(x[n]) if n in c["null"] else x[n]) for n in x}
    O, dO, L, dL = oracle.attention_jvp(xz["q"], xz["k"], xz["v"], xz["dq"], xz["dk"], xz["dv"],
                                        c["scale"], with_dlse=True)
    got = [("O", o, O), ("dO", to, dO)]
    if c["lse"]:
        got.append(("lse", lse, L))
    else:
        assert lse is None
    if c["tlse"]:
        got.append(("tlse", tlse, dL))
    else:
        assert tlse is None
    for name, a, want in got:
        a = a.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(a).all(), (name, c)
        m = metrics(a, want)
        print(f"  [{c['i']}] {name}: {m}", flush=True)
        # bf16 outputs add their own rounding (half an ulp: 2^-9 of the value)
        tol = 2e-2 + (2.0 ** -8 * float(np.abs(want).max()) if c["bf16_out"] and
                      name in ("O", "dO") else 0.0)
        assert m["max_abs"] <= tol, (name, m, c)
        if np.linalg.norm(want) > 0:
            assert m["rel_frob"] <= 1e-2, (name, m, c)


# Forward alone and the backward over a smaller seeded sweep of shapes, each
# with a positive and a negative scale: O, lse against oracle.attention, and
# gQ, gK, gV against oracle.attention_vjp (cotangent gO drawn like dQ), under
# the gates of tests/test_variants.py and tests/test_backward.py.
def _small_configs(n=8, seed=7):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        d = rng.choice([64, 128])
        out.append(dict(i=i, B=rng.choice([1, 2]), H=rng.choice([1, 2]),
                        Nq=rng.choice(EDGES_Q + [rng.randint(1, 700)]),
                        Nk=rng.choice(EDGES_K + [rng.randint(1, 1300)]), d=d))
    return out


@pytest.mark.parametrize("sign", [1.0, -1.0], ids=["pos", "neg"])
@pytest.mark.parametrize("c", _small_configs(), ids=lambda c: (
    f"{c['i']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_forward_and_backward_sweep(c, sign):
    c = dict(c, i=100 + c["i"], tsig=0.1)
    x = _inputs(c)
    s = sign * (0.5 + 0.1 * c["i"] % 7) / math.sqrt(c["d"])
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    print(f"  launch fwd+bwd {c} scale={s:.4f}", flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    gq, gk, gv = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s)
    torch.cuda.synchronize()
    O, L = oracle.attention(x["q"], x["k"], x["v"], s)
    for name, a, want in (("O", o, O), ("lse", lse, L)):
        m = metrics(a.double().cpu().numpy(), want)
        print(f"  [{c['i']}] {name}: {m}", flush=True)
        assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (name, m, c, s)
    ref = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], s)
    for name, a, want in zip(("gQ", "gK", "gV"), (gq, gk, gv), ref):
        a = a.double().cpu().numpy()
        assert np.isfinite(a).all(), (name, c, s)
        m = metrics(a, want)
        print(f"  [{c['i']}] {name}: {m}", flush=True)
        if np.abs(want).max() < 1e-12:  # one key: gQ = gK = 0
            assert m["max_abs"] <= 1e-5, (name, m, c, s)
        else:
            assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2, (name, m, c, s)


@pytest.mark.parametrize("sign", [1.0, -1.0], ids=["pos", "neg"])
@pytest.mark.parametrize("c", _small_configs(n=4, seed=11), ids=lambda c: (
    f"{c['i']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_fp32_path_sweep(c, sign):
    """The fp32 path under both signs of the scale: relative Frobenius <= 1e-5."""
    c = dict(c, i=200 + c["i"], tsig=0.1)
    x = {n: t.float() for n, t in _inputs(c).items()}
    s = sign * 0.9 / math.sqrt(c["d"])
    g = {n: t.to(torch.device("cuda:0")) for n, t in x.items()}
    print(f"  launch fp32 {c} scale={s:.4f}", flush=True)
    o, to, lse = ajvp.attn_jvp_fwd_f32(g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"], scale=s)
    torch.cuda.synchronize()
    ref = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s)
    for name, a, want in zip(("O", "dO", "lse"), (o, to, lse), ref):
        m = metrics(a.double().cpu().numpy(), want)
        print(f"  [{c['i']}] {name}: {m}", flush=True)
        assert m["rel_frob"] <= 1e-5, (name, m, c, s)


# Magnitudes far from 1: every tensor multiplied by its own power of ten
# (V, dV, dQ, dK from 1e-6 to 1e5; Q and K so that the logits stay between
# ~1e-3 and ~30 in size), either sign of the scale, NULL tangents and both
# kernel forms, against the oracle under the scale-free gate of
# tests/test_range.py (relative Frobenius <= 1e-2, max-abs <= 5e-3 of the
# largest reference magnitude).
def _magnitude_configs(n=24, seed=99):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        d = rng.choice([64, 128])
        mq = 10.0 ** rng.uniform(-2, 1)
        mk = 10.0 ** rng.uniform(-1.5, 0.5)
        out.append(dict(
            i=300 + i, B=1, H=rng.choice([1, 2]), Nq=rng.choice(EDGES_Q + [rng.randint(1, 600)]),
            Nk=rng.choice(EDGES_K + [rng.randint(1, 1300)]), d=d,
            scale=rng.choice([1.0, -1.0]) / math.sqrt(d),
            mag=dict(q=mq, k=mk, v=10.0 ** rng.randint(-6, 5), dq=10.0 ** rng.randint(-6, 5),
                     dk=10.0 ** rng.randint(-6, 5), dv=10.0 ** rng.randint(-6, 5)),
            null=rng.choice([(), ("dk", "dv"), ("dq",), ("dv",)]), tsig=1.0))
    return out


@pytest.mark.parametrize("c", _magnitude_configs(), ids=lambda c: (
    f"{c['i']}-q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_magnitude_sweep_vs_oracle(c):
    x = {n: (t.float() * c["mag"][n]).to(torch.bfloat16) for n, t in _inputs(c).items()}
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    tan = {n: (None if n in c["null"] else g[n]) for n in ("dq", "dk", "dv")}
    print(f"  launch magnitudes {c}", flush=True)
    runs = {"plain": ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], tan["dq"], tan["dk"],
                                          tan["dv"], scale=c["scale"]),
            # key-tile ranges merged (3 ranges where the keys span 3 tiles or more)
            "split": ajvp.attn_jvp_fwd_splitkv(g["q"], g["k"], g["v"], tan["dq"], tan["dk"],
                                               tan["dv"], scale=c["scale"], nsplit=3)}
    torch.cuda.synchronize()
    xz = {n: (torch.zeros_like(x[n]) if n in c["null"] else x[n]) for n in x}
    with np.errstate(all="ignore"):
        ref = oracle.attention_jvp(xz["q"], xz["k"], xz["v"], xz["dq"], xz["dk"], xz["dv"],
                                   c["scale"], with_dlse=True)
    for form, outs in runs.items():
        for name, a, want in zip(("O", "dO", "lse", "tlse"), outs, ref):
            a = a.double().cpu().numpy()
            assert np.isfinite(a).all(), (form, name, c)
            m = metrics(a, want)
            print(f"  [{c['i']} {form}] {name}: {m} max|ref| {np.abs(want).max():.3e}",
                  flush=True)
            if np.abs(want).max() == 0:
                assert m["max_abs"] == 0, (form, name, m, c)
                continue
            assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 5e-3, (form, name, m, c)


# The forward alone and the backward with magnitudes far from 1 (per-tensor
# powers of ten; the cotangent gO drawn like dQ and scaled too), either sign
# of the scale, against oracle.attention and oracle.attention_vjp under the
# scale-free gate.
@pytest.mark.parametrize("c", _magnitude_configs(n=16, seed=123), ids=lambda c: (
    f"{c['i']}-q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_magnitude_sweep_forward_and_backward(c):
    c = dict(c, i=c["i"] + 100)
    x = {n: (t.float() * c["mag"][n]).to(torch.bfloat16) for n, t in _inputs(c).items()}
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    s = c["scale"]
    print(f"  launch fwd+bwd magnitudes {c}", flush=True)
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    gq, gk, gv = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        O, L = oracle.attention(x["q"], x["k"], x["v"], s)
        ref = oracle.attention_vjp(x["q"], x["k"], x["v"], x["dq"], s)
    for name, a, want in (("O", o, O), ("lse", lse, L)) + tuple(zip(("gQ", "gK", "gV"),
                                                                    (gq, gk, gv), ref)):
        a = a.double().cpu().numpy()
        assert np.isfinite(a).all(), (name, c)
        m = metrics(a, want)
        print(f"  [{c['i']}] {name}: {m} max|ref| {np.abs(want).max():.3e}", flush=True)
        if np.abs(want).max() < 1e-300:
            continue
        if np.abs(want).max() < 1e-12 * max(1.0, float(np.abs(ref[1]).max())):
            # gQ = gK = 0 up to rounding (a single key): only the size of the result counts
            assert m["max_abs"] <= 1e-5 * max(1.0, float(np.abs(ref[1]).max())), (name, m, c)
            continue
        assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 5e-3, (name, m, c)


# Every entry point that computes the same thing returns the same bits: the
# JVP through the torch workspace (attn_jvp_fwd), the library pool
# (attn_jvp_fwd_ex without a workspace), the two phases (attn_jvp_pack_kv +
# attn_jvp_fwd_packed) and the fixed buffer (attn_jvp_fwd_noalloc); split-KV
# with one range; and the forward alone (its O and lse equal the JVP's).
@pytest.mark.parametrize("c", _configs(n=12, seed=4242), ids=lambda c: (
    f"{c['i']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_entry_points_agree_bit_for_bit(c):
    c = dict(c, i=c["i"] + 500)
    x = _inputs(c)
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    s = c["scale"]
    args = (g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"])
    print(f"  launch entry points {c}", flush=True)
    ref = ajvp.attn_jvp_fwd(*args, scale=s)
    ex = ajvp.attn_jvp_fwd_ex(*args, scale=s, tlse=False)
    ws = torch.empty(ajvp.attn_jvp_workspace_bytes(c["B"], c["H"], c["Nk"], c["d"]),
                     dtype=torch.uint8, device=dev)
    ajvp.attn_jvp_pack_kv(g["k"], g["v"], g["dk"], g["dv"], workspace=ws)
    two = ajvp.attn_jvp_fwd_packed(g["q"], g["dq"], ws, c["Nk"], scale=s)
    na = ajvp.attn_jvp_fwd_noalloc(*args, scale=s)
    sp = ajvp.attn_jvp_fwd_splitkv(*args, scale=s, nsplit=1, tlse=False)
    fo, flse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    torch.cuda.synchronize()
    for name, outs in (("ex", ex[:3]), ("two-phase", two), ("noalloc", na), ("split 1", sp[:3])):
        for a, b, what in zip(outs, ref, ("O", "dO", "lse")):
            assert torch.equal(a, b), (name, what, c)
    assert torch.equal(fo, ref[0]) and torch.equal(flse, ref[2]), c


# Non-finite inputs through every JVP form: one to three NaN or +-Inf values at
# seeded positions of seeded tensors; each output (O, dO, lse, tlse) must be
# non-finite exactly where the oracle's is, and match it elsewhere.
def _nonfinite_configs(n=16, seed=31337):
    rng = random.Random(seed)
    out = []
    for c in _configs(n=n, seed=seed):
        k = rng.randint(1, 3)
        c = dict(c, i=c["i"] + 700, tsig=0.1, bf16_out=False, lse=True, tlse=True,
                 bad=[(rng.choice(["q", "k", "v", "dq", "dk", "dv"]), rng.random(), rng.random(),
                       rng.choice([float("nan"), float("inf"), -float("inf")]))
                      for _ in range(k)])
        out.append(c)
    return out


@pytest.mark.parametrize("c", _nonfinite_configs(), ids=lambda c: (
    f"{c['i']}-B{c['B']}H{c['H']}q{c['Nq']}k{c['Nk']}d{c['d']}"))
def test_nonfinite_sweep_vs_oracle(c):
    x = _inputs(c)
    for name, fr, fc, val in c["bad"]:
        t = x[name]
        b, h = int(fr * 997) % t.shape[0], int(fc * 991) % t.shape[1]
        r, col = int(fr * t.shape[2]) % t.shape[2], int(fc * t.shape[3]) % t.shape[3]
        t[b, h, r, col] = val
    dev = torch.device("cuda:0")
    g = {n: t.to(dev) for n, t in x.items()}
    tan = {n: (None if n in c["null"] else g[n]) for n in ("dq", "dk", "dv")}
    print(f"  launch non-finite {c}", flush=True)
    if c["nsplit"] is None:
        got = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], tan["dq"], tan["dk"], tan["dv"],
                                   scale=c["scale"])
    else:
        got = ajvp.attn_jvp_fwd_splitkv(g["q"], g["k"], g["v"], tan["dq"], tan["dk"], tan["dv"],
                                        scale=c["scale"], nsplit=c["nsplit"])
    torch.cuda.synchronize()
    xz = {n: (torch.zeros_like(x[n]) if n in c["null"] else x[n]) for n in x}
    with np.errstate(all="ignore"):
        ref = oracle.attention_jvp(xz["q"], xz["k"], xz["v"], xz["dq"], xz["dk"], xz["dv"],
                                   c["scale"], with_dlse=True)
    for name, a, want in zip(("O", "dO", "lse", "tlse"), got, ref):
        a = a.double().cpu().numpy()
        bad_g, bad_r = ~np.isfinite(a), ~np.isfinite(want)
        print(f"  [{c['i']}] {name}: {bad_g.sum()} non-finite (oracle {bad_r.sum()})", flush=True)
        assert (bad_g == bad_r).all(), (name, int(bad_g.sum()), int(bad_r.sum()), c)
        if (~bad_r).any():
            m = metrics(a[~bad_r], want[~bad_r])
            assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (name, m, c)
