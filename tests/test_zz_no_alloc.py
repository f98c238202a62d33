"""attn_jvp_fwd_noalloc, the entry point that allocates nothing (GPU).

It runs the kernels of attn_jvp_fwd with the tile images in the library's
fixed device buffer (ATTN_JVP_NOALLOC_BYTES per GPU) instead of a workspace,
so its results must equal attn_jvp_fwd_ws's bit for bit: on two calls in a
row, the second smaller (the buffer keeps the first call's contents), on a
call whose images pass the buffer (run in groups of slices), and after a
frozen-key call through another entry point.
"""

import pytest
import torch

import attention_forward_mode_amd as ajvp

pytestmark = pytest.mark.gpu


def _rand(H, Nq, Nk, seed, d=128):
    g = torch.Generator().manual_seed(seed)
    n = {"q": Nq, "k": Nk, "v": Nk, "dq": Nq, "dk": Nk, "dv": Nk}
    sig = {"q": 1.0, "k": 1.0, "v": 1.0, "dq": 0.1, "dk": 0.1, "dv": 0.1}
    return {name: (torch.randn(1, H, n[name], d, generator=g) * sig[name]).to(torch.bfloat16).cuda()
            for name in n}


def _both(x, label):
    args = [x[n] for n in ("q", "k", "v", "dq", "dk", "dv")]
    print(f"  launch noalloc and ws: {label} q{tuple(x['q'].shape)} k{tuple(x['k'].shape)}",
          flush=True)
    a = ajvp.attn_jvp_fwd_noalloc(*args)
    b = ajvp.attn_jvp_fwd(*args)  # attn_jvp_fwd_ws with a workspace from torch
    torch.cuda.synchronize()
    for u, w, name in zip(a, b, ("O", "dO", "lse")):
        assert torch.isfinite(u).all(), (label, name)
        assert torch.equal(u, w), (label, name)


def test_noalloc_equals_workspace_entry_point():
    _both(_rand(4, 700, 1500, seed=1), "first call")
    _both(_rand(2, 300, 200, seed=2), "second call, smaller")


def test_noalloc_groups_past_its_buffer():
    # 5 slices x 512 key tiles x 64 KiB = 160 MiB of images: groups of 3 and 2
    x = _rand(5, 256, 32768, seed=3)
    _both(x, "past the buffer")


def test_noalloc_after_other_entry_points():
    x = _rand(3, 400, 900, seed=4)
    ajvp.attn_jvp_fwd_ex(x["q"], x["k"], x["v"], x["dq"], None, None)
    ajvp.attn_fwd(x["q"], x["k"], x["v"])
    _both(x, "after frozen-key and forward calls")
