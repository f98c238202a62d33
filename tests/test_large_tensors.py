"""GPU parity for calls whose tensors pass 2^31 bytes.

The kernels address a tensor with 32-bit byte offsets, so the library runs
such a call as consecutive launches over groups of whole (b, h) slices.  Here
B*H = 150 slices of 32760 queries against 100 keys (two 64-key tiles, the
second ragged), d = 128: one slice of an fp32 output is 16.8 MB, so a launch
takes 128 slices and the call runs as groups of 128 and 22 slices; q and tq
are 1.26 GB each in bf16, o and to 2.5 GB each.  Whole slices on both sides of
the group boundary (0, 127, 128, 149) are compared with the fp64 oracle under
the gates of the other parity tests.

Inputs are drawn on the device with seeded generators (on the host the draw
would take minutes) like the image-DiT recipe: Q, K, V N(0, 1), tangents and
the cotangent N(0, 0.1^2); the compared slices are copied back, so the oracle
sees exactly the values the kernels read.
"""

import ctypes

import numpy as np
import pytest
import torch

import attention_forward_mode_amd as ajvp
import oracle

from _gpu import check, metrics

pytestmark = pytest.mark.gpu

B, H, NQ, NK, D = 3, 50, 32760, 100, 128
SCALE = 1.0 / np.sqrt(D)
SLICES = [0, 127, 128, 149]  # first, last of the first group; first, last of the second


def _draw(shape, sigma, seed, dtype):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32)
    return (x * sigma).to(dtype)


def _inputs(dtype=torch.bfloat16):
    q_shape, k_shape = (B, H, NQ, D), (B, H, NK, D)
    x = {
        "q": _draw(q_shape, 1.0, 11, dtype), "k": _draw(k_shape, 1.0, 12, dtype),
        "v": _draw(k_shape, 1.0, 13, dtype), "dq": _draw(q_shape, 0.1, 14, dtype),
        "dk": _draw(k_shape, 0.1, 15, dtype), "dv": _draw(k_shape, 0.1, 16, dtype),
    }
    assert x["q"].numel() * 4 >= 1 << 31  # fp32 outputs past 2^31 bytes
    return x


def _host(t):
    """The compared slices of a [B, H, N, ...] device tensor, as [1, S, N, ...] on the host."""
    flat = t.reshape(B * H, *t.shape[2:])
    return flat[SLICES].cpu().unsqueeze(0)


def _oracle_jvp(x, zero_kv=False):
    h = {n: _host(x[n]) for n in x}
    dk = torch.zeros_like(h["dk"]) if zero_kv else h["dk"]
    dv = torch.zeros_like(h["dv"]) if zero_kv else h["dv"]
    return oracle.attention_jvp(h["q"], h["k"], h["v"], h["dq"], dk, dv, SCALE, with_dlse=True)


def _say(what):
    print(f"  launch {what} B={B} H={H} Nq={NQ} Nk={NK} d={D}", flush=True)


def test_jvp_past_2gib():
    x = _inputs()
    _say("attn_jvp_fwd_ws")
    o, to, lse = ajvp.attn_jvp_fwd(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                   scale=SCALE)
    torch.cuda.synchronize()
    ref_o, ref_do, ref_l, ref_mu = _oracle_jvp(x)
    check("jvp >2GiB", (_host(o), _host(to), _host(lse)), (ref_o, ref_do, ref_l), fp32=False)

    # the entry point with its own (pooled, one group's) workspace: same kernels,
    # same launches, so the same bits
    o2, to2 = torch.empty_like(o), torch.empty_like(to)
    lse2 = torch.empty_like(lse)
    _say("attn_jvp_fwd")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = [ctypes.c_void_p(t.data_ptr()) for t in
         (x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], o2, to2, lse2)]
    rc = ajvp.lib().attn_jvp_fwd(*p, B, H, NQ, NK, D, ctypes.c_float(SCALE), stream)
    assert rc == 0, ajvp.attn_jvp_strerror(rc)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(to2, to) and torch.equal(lse2, lse)
    del o2, to2, lse2

    # the two phases: the pack runs as one group, the fused kernel as two,
    # each finding its slices' tile images at the same place
    _say("attn_jvp_pack_kv + attn_jvp_fwd_packed")
    ws = ajvp.attn_jvp_pack_kv(x["k"], x["v"], x["dk"], x["dv"])
    o3, to3, lse3 = ajvp.attn_jvp_fwd_packed(x["q"], x["dq"], ws, NK, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(to3, to) and torch.equal(lse3, lse)


def test_jvp_ex_frozen_bf16_out_past_2gib():
    x = _inputs()
    _say("attn_jvp_fwd_ex frozen keys, bf16 outputs")
    o, to, lse, mu = ajvp.attn_jvp_fwd_ex(x["q"], x["k"], x["v"], x["dq"], None, None,
                                          scale=SCALE, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref_o, ref_do, ref_l, ref_mu = _oracle_jvp(x, zero_kv=True)
    check("jvp_ex frozen bf16 >2GiB", (_host(o).float(), _host(to).float(), _host(lse)),
          (ref_o, ref_do, ref_l), fp32=False)
    m = metrics(_host(mu).double().numpy(), ref_mu)
    print(f"[jvp_ex frozen bf16 >2GiB] mu: max-abs {m['max_abs']:.3e} "
          f"rel-Frobenius {m['rel_frob']:.3e}", flush=True)
    assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, m


def test_splitkv_past_2gib():
    # nsplit = 2: a 128-slice group's partial O, dO would pass 2^31 bytes, so that
    # group runs unsplit while the 22-slice group runs two key ranges and the merge
    x = _inputs()
    _say("attn_jvp_fwd_splitkv nsplit=2")
    o, to, lse, mu = ajvp.attn_jvp_fwd_splitkv(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                               scale=SCALE, nsplit=2)
    torch.cuda.synchronize()
    ref_o, ref_do, ref_l, ref_mu = _oracle_jvp(x)
    check("splitkv >2GiB", (_host(o), _host(to), _host(lse)), (ref_o, ref_do, ref_l), fp32=False)
    m = metrics(_host(mu).double().numpy(), ref_mu)
    assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, m
    _say("attn_fwd_splitkv nsplit=2")
    o1, l1 = ajvp.attn_fwd_splitkv(x["q"], x["k"], x["v"], scale=SCALE, nsplit=2)
    torch.cuda.synchronize()
    check("fwd splitkv >2GiB", (_host(o1), None, _host(l1)), (ref_o, None, ref_l), fp32=False)


def test_forward_and_backward_past_2gib():
    x = _inputs()
    _say("attn_fwd")
    o, lse = ajvp.attn_fwd(x["q"], x["k"], x["v"], scale=SCALE)
    torch.cuda.synchronize()
    h = {n: _host(x[n]) for n in ("q", "k", "v", "dq")}
    ref_o, ref_l = oracle.attention(h["q"], h["k"], h["v"], SCALE)
    check("fwd >2GiB", (_host(o), None, _host(lse)), (ref_o, None, ref_l), fp32=False)
    _say("attn_bwd")
    gq, gk, gv = ajvp.attn_bwd(x["q"], x["k"], x["v"], o, x["dq"], lse, scale=SCALE)
    torch.cuda.synchronize()
    want = oracle.attention_vjp(h["q"], h["k"], h["v"], h["dq"], SCALE)
    for name, got, ref in zip(("gQ", "gK", "gV"), (gq, gk, gv), want):
        got = _host(got).double().numpy()
        m = metrics(got, ref)
        print(f"[bwd >2GiB] {name}: rel-Frobenius {m['rel_frob']:.3e} "
              f"max-abs/max|ref| {m['max_rel']:.3e}", flush=True)
        assert np.isfinite(got).all(), name
        assert m["rel_frob"] <= 1e-2 and m["max_rel"] <= 2e-2, (name, m)


def test_f32_past_2gib():
    x = _inputs(torch.float32)
    _say("attn_jvp_fwd_f32")
    o, to, lse = ajvp.attn_jvp_fwd_f32(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                       scale=SCALE)
    torch.cuda.synchronize()
    ref_o, ref_do, ref_l, _ = _oracle_jvp(x)
    check("f32 >2GiB", (_host(o), _host(to), _host(lse)), (ref_o, ref_do, ref_l), fp32=True)


@pytest.mark.parametrize("heads,cuts", [
    (138, [64]),                  # R = 4.52M rows: one part's O is 2.3 GB, merged in two row chunks
    (40, [20, 84, 85, 185]),      # 5 parts of 20, 64, 1, 100, 7 keys: parts 3.4 GB in all
])
def test_merge_past_2gib(heads, cuts):
    # the attention of all keys equals the merge of the attentions of a
    # partition of the keys; every part's state comes from attn_jvp_fwd_ex on
    # its keys, the whole from the oracle
    Nk = {138: 128, 40: 192}[heads]
    shape_q, shape_k = (1, heads, NQ, D), (1, heads, Nk, D)
    x = {"q": _draw(shape_q, 1.0, 21, torch.bfloat16), "k": _draw(shape_k, 1.0, 22, torch.bfloat16),
         "v": _draw(shape_k, 1.0, 23, torch.bfloat16), "dq": _draw(shape_q, 0.1, 24, torch.bfloat16),
         "dk": _draw(shape_k, 0.1, 25, torch.bfloat16), "dv": _draw(shape_k, 0.1, 26, torch.bfloat16)}
    bounds = [0, *cuts, Nk]
    P = len(bounds) - 1
    lse_p = torch.empty((P, 1, heads, NQ), dtype=torch.float32, device="cuda:0")
    tlse_p = torch.empty_like(lse_p)
    o_p = torch.empty((P, 1, heads, NQ, D), dtype=torch.float32, device="cuda:0")
    to_p = torch.empty_like(o_p)
    assert o_p.numel() * 4 >= 1 << 31
    for p in range(P):
        a, b = bounds[p], bounds[p + 1]
        kv = {n: x[n][:, :, a:b].contiguous() for n in ("k", "v", "dk", "dv")}
        print(f"  launch attn_jvp_fwd_ex part {p}: keys {a}..{b} H={heads}", flush=True)
        o, to, lse, mu = ajvp.attn_jvp_fwd_ex(x["q"], kv["k"], kv["v"], x["dq"], kv["dk"], kv["dv"],
                                              scale=SCALE)
        o_p[p].copy_(o)
        to_p[p].copy_(to)
        lse_p[p].copy_(lse)
        tlse_p[p].copy_(mu)
        del o, to, lse, mu, kv
    print(f"  launch attn_jvp_merge P={P} R={heads * NQ} d={D}", flush=True)
    lse, o, to, mu = ajvp.attn_jvp_merge(lse_p, o_p, to_p, tlse_p)
    torch.cuda.synchronize()
    del o_p, to_p
    idx = sorted({0, (4194303 // NQ) % heads, heads // 2, heads - 1})
    host = lambda t: t.reshape(heads, *t.shape[2:])[idx].cpu().unsqueeze(0)
    h = {n: host(x[n]) for n in x}
    ref_o, ref_do, ref_l, ref_mu = oracle.attention_jvp(h["q"], h["k"], h["v"], h["dq"], h["dk"],
                                                        h["dv"], SCALE, with_dlse=True)
    check(f"merge P={P} >2GiB", (host(o), host(to), host(lse)), (ref_o, ref_do, ref_l), fp32=False)
    m = metrics(host(mu).double().numpy(), ref_mu)
    assert m["max_abs"] <= 2e-2 and m["rel_frob"] <= 1e-2, m
