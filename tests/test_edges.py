"""GPU edge cases: tiny and ragged sizes, both head dims, degenerate inputs."""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs

from _gpu import check, run, to_device

pytestmark = pytest.mark.gpu

SIZES = [1, 17, 63, 64, 65, 129]


def _rand(B, H, Nq, Nk, d, dtype, seed, tsig=0.1):
    g = torch.Generator().manual_seed(seed)
    r = lambda n, sg=1.0: (torch.randn(B, H, n, d, generator=g) * sg).to(dtype)
    return {"q": r(Nq), "k": r(Nk), "v": r(Nk), "dq": r(Nq, tsig), "dk": r(Nk, tsig),
            "dv": r(Nk, tsig)}


def _cmp(label, x, s):
    outs = run(to_device(x), s)
    refs = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s)
    check(label, outs, refs, fp32=x["q"].dtype == torch.float32)
    return outs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_grid(dtype, d):
    for i, Nq in enumerate(SIZES):
        for j, Nk in enumerate(SIZES):
            x = _rand(1, 2, Nq, Nk, d, dtype, seed=100 * i + j)
            _cmp(f"{dtype} d={d} Nq={Nq} Nk={Nk}", x, 1.0 / math.sqrt(d))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_batches_and_heads_are_independent(dtype):
    """B*H*row-tiles both divisible by 8 (remapped order) and not."""
    for (B, H, Nq) in [(2, 3, 130), (2, 4, 256), (3, 1, 50)]:
        x = _rand(B, H, Nq, 70, 128, dtype, seed=B * 10 + H)
        _cmp(f"{dtype} B={B} H={H} Nq={Nq}", x, 1.0 / math.sqrt(128))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_single_key(dtype):
    """Nk = 1 closed form: P = 1, so O = v0, dO = dv0 (mu equals s dS) and lse = s q.k0.

    The bf16 path rounds s*P*dS to fp16 before the second contraction, so dO
    differs from dv0 by (fp16(s dS) - s dS) v0: at most 2^-11 |s dS| |v0|.
    """
    s = 0.2
    x = _rand(1, 2, 77, 1, 128, dtype, seed=5)
    o, to, lse = _cmp(f"{dtype} Nk=1", x, s)
    q, k, v, dq, dk, dv = (x[n].double() for n in ("q", "k", "v", "dq", "dk", "dv"))
    v0, dv0 = v[:, :, :1].expand(-1, -1, 77, -1), dv[:, :, :1].expand(-1, -1, 77, -1)
    sds = (s * ((dq * k[:, :, :1]).sum(-1) + (q * dk[:, :, :1]).sum(-1))).abs()[..., None]
    u = 1.01 * 2.0 ** -11 if dtype == torch.bfloat16 else 1e-6
    o, to, lse = (t.double().cpu() for t in (o, to, lse))
    assert ((o - v0).abs() <= 1e-6 * v0.abs() + 1e-7).all()
    assert ((to - dv0).abs() <= u * sds * v0.abs() + 1e-6 * (v0.abs() + dv0.abs()) + 1e-7).all()
    lse_ref = s * (q * k[:, :, :1]).sum(-1)
    assert ((lse - lse_ref).abs() <= 1e-6 * (1 + lse_ref.abs())).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_uniform_attention(dtype):
    """Q = 0 (and scale = 0): P = 1/Nk, O = mean of V rows, lse = ln Nk."""
    x = _rand(1, 2, 40, 300, 64, dtype, seed=6)
    x["q"].zero_()
    o, to, lse = _cmp(f"{dtype} Q=0", x, 0.125)
    assert torch.allclose(lse.cpu(), torch.full_like(lse.cpu(), math.log(300)), atol=1e-5)
    y = _rand(1, 2, 40, 300, 64, dtype, seed=7)
    _cmp(f"{dtype} scale=0", y, 0.0)


def test_large_logits():
    """Row max logits up to ~60 (far past the lazy-rescale headroom) and very negative rows."""
    x = _rand(1, 2, 130, 700, 128, torch.bfloat16, seed=8)
    x["q"] = (x["q"].float() * 6.0).to(torch.bfloat16)
    _cmp("bf16 large logits", x, 1.0 / math.sqrt(128))
    y = _rand(1, 1, 64, 200, 64, torch.float32, seed=9)
    y["k"] = y["k"] - 20.0 * y["q"].mean(dim=2, keepdim=True)  # shifts every logit down
    _cmp("fp32 shifted logits", y, 0.125)


def test_increasing_max_along_keys():
    """Key norms grow with the key index, so the running max rises on every tile."""
    x = _rand(1, 1, 128, 1024, 128, torch.bfloat16, seed=10)
    ramp = torch.linspace(0.2, 3.0, 1024)[None, None, :, None]
    x["k"] = (x["k"].float() * ramp).to(torch.bfloat16)
    _cmp("bf16 rising max", x, 1.0 / math.sqrt(128))


def test_cross_frozen_text_reduced():
    x, s = make_inputs("text_cross_frozen", Nq=700, heads=[0, 3])
    _cmp("text_cross_frozen reduced", x, s)


@pytest.mark.parametrize("Nk", [1, 130, 200])
def test_more_row_tiles_than_resident_workgroups(Nk):
    """40 heads x 17 row tiles (the last one ragged) = 680 workgroups, more than
    the chip holds at once (one per CU), in the XCD-aware order; 1, 3 and 4 key
    tiles.  Full JVP with fp32 and bf16 outputs, the frozen-key kernel
    (dK = dV = 0) and the tangent of lse, all against the oracle."""
    import attention_forward_mode_amd as ajvp
    s = 1.0 / math.sqrt(128)
    x = _rand(1, 40, 4100, Nk, 128, torch.bfloat16, seed=Nk)
    _cmp(f"items Nk={Nk}", x, s)
    g = to_device(x)
    print(f"  launch ex frozen/bf16 q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}", flush=True)
    fro = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], None, None, scale=s)
    b16 = ajvp.attn_jvp_fwd_ex(g["q"], g["k"], g["v"], g["dq"], g["dk"], g["dv"], scale=s,
                               out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    zero = torch.zeros_like(x["dk"])
    ref_f = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], zero, zero, s, with_dlse=True)
    check(f"items frozen Nk={Nk}", fro[:3], ref_f[:3], fp32=False)
    # the fourth output is the tangent of lse, mu = rowsum(P * dS) (checked as "O")
    check(f"items frozen tlse Nk={Nk}", (fro[3],), (ref_f[3],), fp32=False)
    ref = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s)
    check(f"items bf16-out Nk={Nk}", b16[:3], ref, fp32=False)


def test_many_small_slices():
    """320 (b, h) slices of 100 query rows and 70 keys: a grid of one row tile
    per slice, more workgroups than CUs, against the oracle."""
    x = _rand(8, 40, 100, 70, 128, torch.bfloat16, seed=11)
    _cmp("B=8 H=40 Nq=100 Nk=70", x, 1.0 / math.sqrt(128))


def test_long_key_sequence():
    """131072 keys (2048 tile images, 128 MiB for the slice) against 300 query
    rows: offsets deep into the workspace slice, checked against the oracle on
    sampled rows."""
    from _gpu import check_sampled
    x = _rand(1, 1, 300, 131072, 128, torch.bfloat16, seed=12)
    s = 1.0 / math.sqrt(128)
    outs = run(to_device(x), s)
    check_sampled("Nq=300 Nk=131072", x, s, outs, rows_per_head=12, extra_rows=(0, 299))
