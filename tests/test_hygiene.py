"""GPU hygiene: every output element is written, results are deterministic,
inputs are left unchanged, both bf16 entry points agree, and invalid calls
launch nothing."""

import ctypes
import math

import pytest
import torch

import attention_forward_mode_amd as ajvp
from workloads import make_inputs

from _gpu import NAMES, to_device

pytestmark = pytest.mark.gpu


def _inputs(dtype=torch.bfloat16):
    name = "image_dit" if dtype == torch.bfloat16 else "tiny_fp32"
    x, s = make_inputs(name, Nq=333, Nk=271, heads=[0, 1, 2])
    return to_device(x), s


def _fn(g):
    return ajvp.attn_jvp_fwd if g["q"].dtype == torch.bfloat16 else ajvp.attn_jvp_fwd_f32


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_every_output_written(dtype):
    g, s = _inputs(dtype)
    B, H, Nq, d = g["q"].shape
    o = torch.full((B, H, Nq, d), float("nan"), device="cuda")
    to = torch.full_like(o, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device="cuda")
    _fn(g)(*[g[n] for n in NAMES], scale=s, out=(o, to, lse))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(to).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_deterministic_and_inputs_unchanged(dtype):
    g, s = _inputs(dtype)
    before = {n: g[n].clone() for n in NAMES}
    a = _fn(g)(*[g[n] for n in NAMES], scale=s)
    b = _fn(g)(*[g[n] for n in NAMES], scale=s)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for n in NAMES:
        assert torch.equal(before[n], g[n])


def test_lse_optional():
    g, s = _inputs()
    o1, t1, _ = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s, lse=True)
    o2, t2, l2 = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s, lse=False)
    torch.cuda.synchronize()
    assert l2 is None and torch.equal(o1, o2) and torch.equal(t1, t2)


def test_pool_entry_point_matches_workspace_entry_point():
    """attn_jvp_fwd (library-owned stream-ordered workspace) == attn_jvp_fwd_ws."""
    g, s = _inputs()
    o1, t1, l1 = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)
    o2, t2, l2 = torch.empty_like(o1), torch.empty_like(t1), torch.empty_like(l1)
    B, H, Nq, d = g["q"].shape
    Nk = g["k"].shape[2]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):  # second call reuses the pooled workspace
        rc = ajvp.lib().attn_jvp_fwd(*[p(g[n]) for n in NAMES], p(o2), p(t2), p(l2), B, H, Nq,
                                     Nk, d, ctypes.c_float(s), stream)
        assert rc == 0, ajvp.attn_jvp_strerror(rc)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(t1, t2) and torch.equal(l1, l2)


def test_pool_entry_point_from_two_threads():
    """attn_jvp_fwd called from two host threads at once, each on its own
    stream (default priority), each taking its workspace from the library's
    pool: every call equals attn_jvp_fwd_ws's result bit for bit."""
    import threading

    cases = []
    for seed, (Nq, Nk) in enumerate([(333, 1500), (700, 271)]):
        x, s = make_inputs("image_dit", Nq=Nq, Nk=Nk, heads=[seed, seed + 1])
        g = to_device(x)
        ref = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)  # caller workspace (_ws)
        outs = [tuple(torch.empty_like(t) for t in ref) for _ in range(4)]
        cases.append((g, s, ref, outs))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    start = threading.Barrier(2)
    rcs = [[], []]
    p = lambda t: ctypes.c_void_p(t.data_ptr())

    def work(i):
        g, s, _, outs = cases[i]
        B, H, Nq, d = g["q"].shape
        st = ctypes.c_void_p(streams[i].cuda_stream)
        start.wait()
        for o, to, lse in outs:
            rcs[i].append(ajvp.lib().attn_jvp_fwd(*[p(g[n]) for n in NAMES], p(o), p(to), p(lse),
                                                  B, H, Nq, g["k"].shape[2], d, ctypes.c_float(s),
                                                  st))

    print("  launch attn_jvp_fwd from two threads on two streams", flush=True)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert rcs == [[0] * 4, [0] * 4], rcs
    for g, s, ref, outs in cases:
        for out in outs:
            for a, b in zip(out, ref):
                assert torch.equal(a, b)


def test_rejected_call_leaves_outputs_untouched():
    g, s = _inputs()
    B, H, Nq, d = g["q"].shape
    o = torch.full((B, H, Nq, d), 7.0, device="cuda")
    to = torch.full_like(o, 7.0)
    lse = torch.full((B, H, Nq), 7.0, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = ajvp.lib().attn_jvp_fwd(*[p(g[n]) for n in NAMES], p(o), p(to), p(lse), B, H, Nq,
                                 g["k"].shape[2], 96, ctypes.c_float(s), stream)
    assert rc == -2
    rc = ajvp.lib().attn_jvp_fwd(*[p(g[n]) for n in NAMES], p(o), p(to), p(lse), B, H, Nq,
                                 g["k"].shape[2], d, ctypes.c_float(float("nan")), stream)
    assert rc == -1
    torch.cuda.synchronize()
    assert (o == 7).all() and (to == 7).all() and (lse == 7).all()


def test_python_binding_validation():
    g, s = _inputs()
    with pytest.raises(ValueError):
        ajvp.attn_jvp_fwd(g["q"].float(), *[g[n] for n in NAMES[1:]])
    with pytest.raises(ValueError):
        ajvp.attn_jvp_fwd(g["q"], g["k"][:, :, :10], *[g[n] for n in NAMES[2:]])
    with pytest.raises(ValueError):
        ajvp.attn_jvp_fwd(g["q"].transpose(2, 3), *[g[n] for n in NAMES[1:]])
    # a host workspace never reaches the kernels
    with pytest.raises(ValueError):
        ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ajvp.attn_jvp_pack_kv(g["k"], g["v"], g["dk"], g["dv"],
                              workspace=torch.empty(1 << 20, dtype=torch.uint8))


def test_two_phases_match_fused_and_packed_workspace_is_reusable():
    """attn_jvp_pack_kv + attn_jvp_fwd_packed == attn_jvp_fwd bit for bit; one
    packed K/V/dK/dV serves two query batches of different lengths."""
    g, s = _inputs()
    ref = ajvp.attn_jvp_fwd(*[g[n] for n in NAMES], scale=s)
    ws = ajvp.attn_jvp_pack_kv(g["k"], g["v"], g["dk"], g["dv"])
    Nk = g["k"].shape[2]
    got = ajvp.attn_jvp_fwd_packed(g["q"], g["dq"], ws, Nk, scale=s)
    q2, dq2 = g["q"][:, :, :97].contiguous(), g["dq"][:, :, :97].contiguous()
    got2 = ajvp.attn_jvp_fwd_packed(q2, dq2, ws, Nk, scale=s)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    for a, b in zip(ref, got2):
        assert torch.equal(a[:, :, :97], b)
