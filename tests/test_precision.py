"""Precision of the attention layer's tangent, measured (GPU).

The rCM pages report that a JVP computed in BF16 loses far more accuracy than
an output computed in BF16 (Anthology of the SOTA, LIT-783, "Key takeaways",
Fig. 11), and
that a finite difference of the time derivative with dt = 1e-4 replaces the
JVP only for the smallest model (§4.2).  This measures both at the level of
one attention layer on each workload shape (first head, full length): the
relative Frobenius error, against the fp64 oracle on the unrounded fp32 draws,
of

  * O and dO from the bf16 kernel (inputs rounded to bf16), and the same
    against the oracle on the rounded inputs (the kernel's own arithmetic),
  * O and dO from the fp32 kernel,
  * dO from a central finite difference of the forward kernels,
    (attn(x + h t) - attn(x - h t)) / 2h, in bf16 (perturbed inputs rounded to
    bf16, as a bf16 network holds them) and in fp32, for h = 1e-4 and 1e-2,

and prints the table.  What it shows (and asserts): at one layer the bf16
tangent's relative error is of the same size as the output's (both set by the
rounding of the inputs, not by the kernel), so the model-level gap the pages
report has to build up elsewhere; fp32 removes nearly all of it; a bf16 finite
difference at h = 1e-4 loses the tangent entirely, and even an fp32 one is
orders of magnitude worse than the JVP."""

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle
from workloads import make_inputs

from _gpu import NAMES

pytestmark = pytest.mark.gpu

WORKLOADS = ["image_dit", "text_cross_frozen", "text_cross", "video_1p3b", "video_14b"]


def _rel(got, want):
    got = np.asarray(got, dtype=np.float64)
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


@pytest.mark.parametrize("name", WORKLOADS)
def test_tangent_precision(name):
    x32, s = make_inputs(name, heads=[0], dtype="fp32")
    g32 = {n: t.cuda() for n, t in x32.items()}
    g16 = {n: t.to(torch.bfloat16) for n, t in g32.items()}
    Nq = x32["q"].shape[2]
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(Nq, 48, replace=False), [0, Nq - 1]]))
    O, dO, _ = oracle.attention_jvp_rows(x32["q"], x32["k"], x32["v"], x32["dq"], x32["dk"],
                                         x32["dv"], s, 0, 0, rows)
    x16 = {n: t.to(torch.bfloat16) for n, t in x32.items()}
    O16, dO16, _ = oracle.attention_jvp_rows(x16["q"], x16["k"], x16["v"], x16["dq"], x16["dk"],
                                             x16["dv"], s, 0, 0, rows)
    pick = lambda t: t[0, 0, rows].double().cpu().numpy()

    print(f"  launch precision study {name}", flush=True)
    ob, dob, _ = ajvp.attn_jvp_fwd(*[g16[n] for n in NAMES], scale=s)
    of, dof, _ = ajvp.attn_jvp_fwd_f32(*[g32[n] for n in NAMES], scale=s)
    res = {"O bf16": _rel(pick(ob), O), "dO bf16": _rel(pick(dob), dO),
           "O bf16 kernel": _rel(pick(ob), O16), "dO bf16 kernel": _rel(pick(dob), dO16),
           "O fp32": _rel(pick(of), O), "dO fp32": _rel(pick(dof), dO)}
    zero = {n: torch.zeros_like(g32[n]) for n in ("dq", "dk", "dv")}
    for h in (1e-4, 1e-2):
        side = {}
        for sign in (1, -1):
            xp = {n: g32[n] + sign * h * g32["d" + n] for n in ("q", "k", "v")}
            side[("bf16", sign)] = ajvp.attn_fwd(*[xp[n].to(torch.bfloat16) for n in ("q", "k", "v")],
                                                 scale=s)[0]
            side[("fp32", sign)] = ajvp.attn_jvp_fwd_f32(xp["q"], xp["k"], xp["v"], zero["dq"],
                                                         zero["dk"], zero["dv"], scale=s)[0]
        for prec in ("bf16", "fp32"):
            fd = (side[(prec, 1)] - side[(prec, -1)]) / (2 * h)
            res[f"FD {prec} h={h:g}"] = _rel(pick(fd), dO)
    torch.cuda.synchronize()
    print(f"[precision {name}] " + "  ".join(f"{k}: {v:.3e}" for k, v in res.items()), flush=True)
    assert all(np.isfinite(v) for v in res.values())
    # one layer: the bf16 tangent's relative error is of the output's size
    assert 0.3 * res["O bf16"] < res["dO bf16"] < 3 * res["O bf16"]
    # ... and set by the rounding of the inputs: the kernel's own arithmetic
    # adds less than the rounding does
    assert res["O bf16 kernel"] < res["O bf16"] and res["dO bf16 kernel"] < res["dO bf16"]
    # fp32 arithmetic on unrounded inputs removes nearly all of it
    assert res["dO fp32"] < 0.01 * res["dO bf16"]
    # finite differences: at h = 1e-4 a bf16 one loses the tangent, and an fp32
    # one is orders of magnitude worse than the JVP
    assert res["FD bf16 h=0.0001"] > 1.0
    assert res["FD fp32 h=0.0001"] > 100 * res["dO fp32"]
