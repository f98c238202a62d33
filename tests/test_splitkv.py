"""GPU tests of the split-KV entry point: key-tile ranges on separate
workgroups, partial (lse, O, dO, mu) states merged.  One range equals the
unsplit kernel bit for bit; several ranges pass the oracle gate (outputs and
the tangent of lse), for ragged key counts, the frozen-key kernel and a
short-query / long-key shape at full key length."""

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle
from workloads import make_inputs

from _gpu import NAMES, check, to_device

pytestmark = pytest.mark.gpu


def _split(g, s, nsplit, frozen=False):
    tk, tv = (None, None) if frozen else (g["dk"], g["dv"])
    print(f"  launch splitkv nsplit={nsplit} frozen={frozen} q{tuple(g['q'].shape)} "
          f"k{tuple(g['k'].shape)}", flush=True)
    out = ajvp.attn_jvp_fwd_splitkv(g["q"], g["k"], g["v"], g["dq"], tk, tv, scale=s,
                                    nsplit=nsplit)
    torch.cuda.synchronize()
    return out


def test_one_range_is_the_unsplit_kernel():
    x, s = make_inputs("image_dit", Nq=333, Nk=2000, heads=[0, 1])
    g = to_device(x)
    a = _split(g, s, 1)
    b = ajvp.attn_jvp_fwd_ex(*[g[n] for n in NAMES], scale=s)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("Nq,Nk,nsplit", [(1, 5000, 0), (100, 1000, 3), (100, 1000, 5),
                                          (77, 4097, 16), (300, 700, 0), (64, 64, 4)])
@pytest.mark.parametrize("frozen", [False, True])
def test_split_ranges_against_oracle(Nq, Nk, nsplit, frozen):
    x, s = make_inputs("video_1p3b", Nq=Nq, Nk=Nk, heads=[0, 1])
    g = to_device(x)
    o, to, lse, tlse = _split(g, s, nsplit, frozen)
    dk, dv = (np.zeros(x["dk"].shape), np.zeros(x["dv"].shape)) if frozen else (x["dk"], x["dv"])
    O, dO, L, MU = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], dk, dv, s, with_dlse=True)
    label = f"split Nq={Nq} Nk={Nk} n={nsplit} frozen={frozen}"
    check(label, (o, to, lse), (O, dO, L), fp32=False)
    check(label + " tlse", (tlse,), (MU,), fp32=False)


def test_short_queries_long_keys_full_length():
    """256 query rows of 12 heads against all 32760 keys (12 workgroups
    unsplit): the automatic split, sampled rows of every head against the
    oracle."""
    x, s = make_inputs("video_1p3b", Nq=256)
    g = to_device(x)
    o, to, lse, tlse = _split(g, s, 0)
    rows = [0, 1, 100, 128, 255]
    got = [[], [], []]
    ref = [[], [], []]
    for h in range(12):
        O, dO, L = oracle.attention_jvp_rows(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                             s, 0, h, rows)
        for i, (t, r) in enumerate(zip((o, to, lse), (O, dO, L))):
            got[i].append(t[0, h, rows].double().cpu().numpy())
            ref[i].append(r)
    check("split 256 x 32760 H12 auto", tuple(np.concatenate(a) for a in got),
          tuple(np.concatenate(r) for r in ref), fp32=False)


def test_forward_one_range_is_attn_fwd():
    x, s = make_inputs("image_dit", Nq=333, Nk=2000, heads=[0, 1])
    g = to_device(x)
    print("  launch attn_fwd_splitkv nsplit=1 / attn_fwd", flush=True)
    a = ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=s, nsplit=1)
    b = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("Nq,Nk,nsplit", [(1, 5000, 0), (100, 1000, 3), (77, 4097, 16),
                                          (600, 2000, 0)])
def test_forward_split_ranges_against_oracle(Nq, Nk, nsplit):
    x, s = make_inputs("video_14b", Nq=Nq, Nk=Nk, heads=[0, 1])
    g = to_device(x)
    print(f"  launch attn_fwd_splitkv nsplit={nsplit} Nq={Nq} Nk={Nk}", flush=True)
    o, lse = ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=s, nsplit=nsplit)
    torch.cuda.synchronize()
    O, L = oracle.attention(x["q"], x["k"], x["v"], s)
    check(f"fwd split Nq={Nq} Nk={Nk} n={nsplit}", (o, None, lse), (O, None, L), fp32=False)
