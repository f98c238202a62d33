"""The forms of the bf16 kernels against each other and the oracle (GPU).

The JVP has a 256-row kernel and a 128-row short-key kernel (two workgroups
per CU), chosen by the number of key tiles per work item; the forward pass
alone has 512-row (two 32-row blocks per wave) and 256-row forms.  Each form
computes every row with the same products in the same order, so the results
must be equal bit for bit whichever form runs (ATTN_JVP_TILE forces one).  The
256-row JVP kernel's frozen-key, bf16-output and d = 64 instances are also
checked against the oracle with more than 16 key tiles, where the automatic
choice takes them."""

import math
import os

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle

from _gpu import metrics

pytestmark = pytest.mark.gpu


def _rand(H, Nq, Nk, d, seed):
    g = torch.Generator().manual_seed(seed)
    n = {"q": Nq, "k": Nk, "v": Nk, "dq": Nq, "dk": Nk, "dv": Nk}
    sig = {"q": 1.0, "k": 1.0, "v": 1.0, "dq": 0.1, "dk": 0.1, "dv": 0.1}
    return {name: (torch.randn(1, H, n[name], d, generator=g) * sig[name]).to(torch.bfloat16)
            for name in n}


def _with_tile(tile, fn):
    old = os.environ.get("ATTN_JVP_TILE")
    os.environ["ATTN_JVP_TILE"] = str(tile)
    try:
        out = fn()
        torch.cuda.synchronize()
        return [None if t is None else t.cpu() for t in out]
    finally:
        if old is None:
            del os.environ["ATTN_JVP_TILE"]
        else:
            os.environ["ATTN_JVP_TILE"] = old


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nk", [300, 1500])
@pytest.mark.parametrize("mode", ["full", "frozen", "bf16_out"])
def test_jvp_forms_agree(mode, Nk, d):
    x = _rand(2, 333, Nk, d, seed=Nk + d)
    g = {n: t.cuda() for n, t in x.items()}
    s = 1.0 / math.sqrt(d)
    frozen = mode == "frozen"
    out_dtype = torch.bfloat16 if mode == "bf16_out" else torch.float32

    def call():
        print(f"  launch jvp_ex {mode} Nk={Nk} d={d} tile={os.environ['ATTN_JVP_TILE']}",
              flush=True)
        return ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], None if frozen else g["dk"],
                                    None if frozen else g["dv"], scale=s, out_dtype=out_dtype)
    a = _with_tile(128, call)
    b = _with_tile(256, call)
    for u, w, name in zip(a, b, ("O", "dO", "lse", "mu")):
        assert torch.equal(u, w), (mode, Nk, d, name)


@pytest.mark.parametrize("Nk", [300, 1500])
def test_forward_forms_agree_with_each_other_and_the_jvp(Nk):
    x = _rand(2, 700, Nk, 128, seed=7 * Nk)
    g = {n: t.cuda() for n, t in x.items()}
    s = 1.0 / math.sqrt(128)

    def fwd():
        return ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    a = _with_tile(256, fwd)
    b = _with_tile(512, fwd)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o, _, lse = ajvp.attn_jvp_fwd(g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"], scale=s)
    torch.cuda.synchronize()
    assert torch.equal(a[0], o.cpu()) and torch.equal(a[1], lse.cpu())


@pytest.mark.parametrize("mode,d", [("frozen", 128), ("bf16_out", 128), ("full", 64),
                                    ("frozen", 64)])
def test_256_row_kernel_instances_vs_oracle(mode, d):
    """More than 16 key tiles (1500 keys, a ragged last tile): the 256-row
    kernel, in the instances that the short-key tests do not reach."""
    x = _rand(2, 300, 1500, d, seed=11 + d)
    g = {n: t.cuda() for n, t in x.items()}
    s = 1.0 / math.sqrt(d)
    frozen = mode == "frozen"
    out_dtype = torch.bfloat16 if mode == "bf16_out" else torch.float32
    print(f"  launch jvp_ex {mode} d={d} q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}", flush=True)
    o, to, lse, mu = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"],
                                          None if frozen else g["dk"], None if frozen else g["dv"],
                                          scale=s, out_dtype=out_dtype)
    torch.cuda.synchronize()
    z = torch.zeros_like(x["dk"])
    O, dO, L, MU = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], z if frozen else x["dk"],
                                        z if frozen else x["dv"], s, with_dlse=True)
    for name, got, want in (("O", o, O), ("dO", to, dO), ("lse", lse, L), ("mu", mu, MU)):
        m = metrics(got.double().cpu().numpy(), want)
        print(f"[{mode} d={d}] {name}: max-abs {m['max_abs']:.3e} rel-Frobenius "
              f"{m['rel_frob']:.3e}", flush=True)
        assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (mode, d, name, m)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nk", [30, 100, 130])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_forward_512_row_form_on_few_tiles(Nk, d, out_dtype):
    """The 512-row forward form runs its two wave groups a phase apart over
    three rotating tile stages; with 1, 2 and 3 key tiles (ragged last tile)
    its first and last tiles meet (no previous tile, no next one).  Forced by
    ATTN_JVP_TILE, it must equal the 256-row form bit for bit, and the oracle
    within the gate; split ranges of 1-2 tiles likewise."""
    x = _rand(2, 1100, Nk, d, seed=3 * Nk + d)
    g = {n: t.cuda() for n, t in x.items()}
    s = 1.0 / math.sqrt(d)

    def fwd():
        print(f"  launch attn_fwd Nk={Nk} d={d} {out_dtype} tile={os.environ['ATTN_JVP_TILE']}",
              flush=True)
        return ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s, out_dtype=out_dtype)
    a = _with_tile(256, fwd)
    b = _with_tile(512, fwd)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (Nk, d)
    z = torch.zeros_like(x["q"])
    O, _, L = oracle.attention_jvp(x["q"], x["k"], x["v"], z, torch.zeros_like(x["k"]),
                                   torch.zeros_like(x["v"]), s)[:3]
    for name, got, want in (("O", b[0], O), ("lse", b[1], L)):
        m = metrics(got.double().numpy(), want)
        assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (Nk, d, name, m)
    if out_dtype == torch.float32 and Nk > 64:
        for ns in (2, (Nk + 63) // 64):
            def split():
                print(f"  launch attn_fwd_splitkv Nk={Nk} d={d} nsplit={ns} "
                      f"tile={os.environ['ATTN_JVP_TILE']}", flush=True)
                return ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=s, nsplit=ns)
            c = _with_tile(256, split)
            e = _with_tile(512, split)
            assert torch.equal(c[0], e[0]) and torch.equal(c[1], e[1]), (Nk, d, ns)
            m = metrics(e[0].double().numpy(), O)
            assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, (Nk, d, ns, m)
