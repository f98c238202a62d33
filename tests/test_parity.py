"""GPU parity: the HIP path against the fp64 oracle on the seeded workloads.

Gate (from the target's statement): bf16 inputs with fp32 accumulation must
match within max-abs <= 2e-2 and relative Frobenius <= 1e-2 on O and dO (lse
is held to the same bounds); the fp32 path within relative Frobenius <= 1e-5.
Small cases compare every element; the full-size workloads run in the launch
configuration the benchmark times and compare sampled rows (rows are
independent) plus properties of every row.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, outlier_rows

from _gpu import check, check_sampled, run, to_device

pytestmark = pytest.mark.gpu


def _full(label, x, s):
    g = to_device(x)
    outs = run(g, s)
    refs = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s)
    check(label, outs, refs, fp32=x["q"].dtype == torch.float32)


def test_tiny_fp32_full():
    """fp32 self-attention B=1 H=2 N=256 d=64: every element."""
    x, s = make_inputs("tiny_fp32")
    _full("tiny_fp32", x, s)


@pytest.mark.parametrize("Nq,Nk", [(256, 256), (300, 200), (129, 515), (1000, 64), (64, 1000)])
def test_image_dit_reduced_full(Nq, Nk):
    """bf16 image-DiT recipe at sizes that span several tiles and ragged tails."""
    x, s = make_inputs("image_dit", Nq=Nq, Nk=Nk, heads=[0, 5, 9])
    _full(f"image_dit {Nq}x{Nk}", x, s)


@pytest.mark.parametrize("name", ["video_1p3b", "video_14b"])
def test_video_recipes_reduced_full(name):
    """The video recipes (row-max placement, x8 outliers) at 1000 x 1500, every element."""
    x, s = make_inputs(name, Nq=1000, Nk=1500, heads=[0, 1])
    _full(f"{name} reduced", x, s)


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_ragged_full(d):
    x, s = make_inputs("tiny_fp32", Nq=333, Nk=97, heads=[0, 1])
    if d == 128:
        x = {n: torch.cat([t, t.flip(-1)], dim=-1).contiguous() for n, t in x.items()}
        s = 1.0 / np.sqrt(128)
    _full(f"fp32 d={d} 333x97", x, s)


@pytest.mark.slow
def test_image_dit_full_size():
    x, s = make_inputs("image_dit")
    outs = run(to_device(x), s)
    check_sampled("image_dit B2 H16 N4096", x, s, outs, rows_per_head=16)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["text_cross_frozen", "text_cross"])
def test_text_cross_full_size(name):
    x, s = make_inputs(name)
    outs = run(to_device(x), s)
    check_sampled(f"{name} H12 32760x512", x, s, outs, rows_per_head=32)


@pytest.mark.slow
def test_video_1p3b_full_size():
    x, s = make_inputs("video_1p3b")
    outs = run(to_device(x), s)
    check_sampled("video_1p3b H12 N32760", x, s, outs, rows_per_head=24)


@pytest.mark.slow
def test_video_14b_full_size():
    w = WORKLOADS["video_14b"]
    x, s = make_inputs("video_14b")
    outs = run(to_device(x), s)
    q_out = outlier_rows(0, 0, w.Nq, w.outlier_frac)[:4].tolist()
    check_sampled("video_14b H40 N32760", x, s, outs, rows_per_head=12, extra_rows=q_out)


@pytest.mark.slow
def test_video_14b_head_shard_full_size():
    """One GPU's share of the 14B shape under an 8-way head split (H = 5), in
    the launch configuration bench.py times for it."""
    w = WORKLOADS["video_14b_shard8"]
    x, s = make_inputs("video_14b_shard8")
    outs = run(to_device(x), s)
    q_out = outlier_rows(0, 0, w.Nq, w.outlier_frac)[:4].tolist()
    check_sampled("video_14b_shard8 H5 N32760", x, s, outs, rows_per_head=24, extra_rows=q_out)


@pytest.mark.slow
def test_video_14b_fp32_full_size():
    x, s = make_inputs("video_14b_fp32")
    outs = run(to_device(x), s)
    check_sampled("video_14b_fp32 H2 N32760", x, s, outs, rows_per_head=24)
