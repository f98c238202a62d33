"""HIP graph capture of the entry points that allocate nothing (caller
workspace and outputs): the captured launches replay to the eager result,
replay after replay, with eager work and synchronisations in between, and
follow new values written into the captured input buffers.  None of the
library's launches is a memset or a copy, so a captured graph holds kernel
nodes only."""

import pytest
import torch

import attention_forward_mode_amd as ajvp
from workloads import make_inputs

from _gpu import NAMES, to_device

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm up on a side stream (default priority), then capture fn()."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _replays_match(graph, outs, want, n=3):
    for i in range(n):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {i}"


def test_jvp_graph_replays():
    x, s = make_inputs("image_dit", Nq=700, Nk=900, heads=[0, 1])
    g = to_device(x)
    B, H, Nq, d = g["q"].shape
    Nk = g["k"].shape[2]
    ws = torch.empty(ajvp.attn_jvp_workspace_bytes(B, H, Nk, d), dtype=torch.uint8, device="cuda")
    outs = tuple(torch.empty(sh, dtype=torch.float32, device="cuda")
                 for sh in ((B, H, Nq, d), (B, H, Nq, d), (B, H, Nq)))
    args = [g[n] for n in NAMES]
    print(f"  capture attn_jvp_fwd q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}", flush=True)
    graph = _capture(lambda: ajvp.attn_jvp_fwd(*args, scale=s, out=outs, workspace=ws))
    want = ajvp.attn_jvp_fwd(*args, scale=s)
    torch.cuda.synchronize()
    _replays_match(graph, outs, want)
    # new values in the captured input buffers
    x2, _ = make_inputs("image_dit", seed=1, Nq=700, Nk=900, heads=[0, 1])
    for n in NAMES:
        g[n].copy_(x2[n].to("cuda"))
    want2 = ajvp.attn_jvp_fwd(*args, scale=s)
    torch.cuda.synchronize()
    assert not torch.equal(want2[0], want[0])
    _replays_match(graph, outs, want2)


def test_forward_and_backward_graph_replays():
    x, s = make_inputs("image_dit", Nq=600, Nk=300, heads=[0, 1, 2])
    g = to_device(x)
    B, H, Nq, d = g["q"].shape
    Nk = g["k"].shape[2]
    ws = torch.empty(max(ajvp.attn_jvp_workspace_bytes(B, H, Nk, d),
                         ajvp.attn_bwd_workspace_bytes(B, H, Nq, Nk, d)),
                     dtype=torch.uint8, device="cuda")
    o, lse = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s)
    want = ajvp.attn_bwd(g["q"], g["k"], g["v"], o, g["dq"], lse, scale=s)
    torch.cuda.synchronize()
    print(f"  capture attn_fwd + attn_bwd q{tuple(g['q'].shape)} k{tuple(g['k'].shape)}",
          flush=True)
    state = {}

    def step():
        state["fwd"] = ajvp.attn_fwd(g["q"], g["k"], g["v"], scale=s, workspace=ws)
        fo, fl = state["fwd"]
        state["bwd"] = ajvp.attn_bwd(g["q"], g["k"], g["v"], fo, g["dq"], fl, scale=s,
                                     workspace=ws)

    graph = _capture(step)
    outs = tuple(state["fwd"]) + tuple(state["bwd"])
    _replays_match(graph, outs, (o, lse) + tuple(want))


def test_splitkv_graph_replays():
    # few queries against many keys: key ranges on separate workgroups, then
    # the merge kernel, all in the captured graph (caller workspace)
    x, s = make_inputs("image_dit", Nq=100, Nk=5000, heads=[0, 1])
    g = to_device(x)
    B, H, Nq, d = g["q"].shape
    Nk = g["k"].shape[2]
    nb = max(ajvp.attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0),
             ajvp.attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, 7))
    assert nb > ajvp.attn_jvp_workspace_bytes(B, H, Nk, d)  # partial states: more than one range
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    args = [g[n] for n in NAMES]
    want = ajvp.attn_jvp_fwd_splitkv(*args, scale=s)
    want_f = ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=s, nsplit=7)
    torch.cuda.synchronize()
    print(f"  capture attn_jvp_fwd_splitkv + attn_fwd_splitkv q{tuple(g['q'].shape)} "
          f"k{tuple(g['k'].shape)}", flush=True)
    state = {}

    def step():
        state["jvp"] = ajvp.attn_jvp_fwd_splitkv(*args, scale=s, workspace=ws)
        state["fwd"] = ajvp.attn_fwd_splitkv(g["q"], g["k"], g["v"], scale=s, nsplit=7,
                                             workspace=ws)

    graph = _capture(step)
    outs = tuple(state["jvp"]) + tuple(state["fwd"])
    _replays_match(graph, outs, tuple(want) + tuple(want_f))
