"""The seeded input recipe: determinism, structure and value ranges (CPU only)."""

import math

import numpy as np
import torch

from workloads import TENSORS, WORKLOADS, make_inputs, outlier_rows


def test_deterministic_and_head_subsets():
    a, s1 = make_inputs("image_dit", Nq=64, Nk=96)
    b, s2 = make_inputs("image_dit", Nq=64, Nk=96)
    c, _ = make_inputs("image_dit", Nq=64, Nk=96, heads=[3, 7])
    assert s1 == s2 == 1.0 / math.sqrt(128)
    for t in TENSORS:
        assert torch.equal(a[t], b[t])
        assert torch.equal(a[t][:, [3, 7]], c[t])
        assert a[t].is_contiguous() and a[t].dtype == torch.bfloat16
    assert a["q"].shape == (2, 16, 64, 128) and a["k"].shape == (2, 16, 96, 128)
    d, _ = make_inputs("image_dit", seed=1, Nq=64, Nk=96)
    assert not torch.equal(a["q"], d["q"])


def test_sigmas():
    x, _ = make_inputs("image_dit", Nq=512, Nk=512, heads=[0])
    for t, want in zip(TENSORS, (1.0, 1.0, 1.0, 0.1, 0.1, 0.1)):
        sd = x[t].float().std().item()
        assert abs(sd - want) < 0.05 * want, (t, sd)


def test_bf16_is_round_to_nearest_even():
    g = torch.Generator().manual_seed(11)
    f = torch.randn(4096, generator=g)
    bits = f.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    # round-to-nearest-even on the upper 16 bits, by integer arithmetic
    lsb = (bits >> 16) & 1
    rne = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    got = f.to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(got, rne)


def test_frozen_text_tangents_are_zero():
    x, _ = make_inputs("text_cross_frozen", Nq=100, heads=[0, 5])
    assert x["dk"].abs().max() == 0 and x["dv"].abs().max() == 0
    assert x["dq"].abs().max() > 0
    y, _ = make_inputs("text_cross", Nq=100, heads=[0, 5])
    assert torch.equal(x["q"], y["q"]) and torch.equal(x["k"], y["k"])
    assert y["dk"].abs().max() > 0


def test_row_max_placement_reduced():
    """Row maxima of scale * q.k land in [5, 20] (up to bf16 rounding of q)."""
    x, s = make_inputs("video_1p3b", Nq=300, Nk=2048, heads=[0, 11], device="cpu")
    for hi in range(2):
        q = x["q"][0, hi].double()
        k = x["k"][0, hi].double()
        m = s * (q @ k.T).max(dim=1).values
        assert m.min() >= 5.0 * (1 - 2 ** -7) and m.max() <= 20.0 * (1 + 2 ** -7), (m.min(), m.max())
        assert m.max() - m.min() > 10.0  # spread over the range, not collapsed


def test_outliers():
    w = WORKLOADS["video_14b"]
    idx = outlier_rows(0, 1, w.Nk, w.outlier_frac)
    assert len(idx) == 328 and len(set(idx.tolist())) == 328
    x, _ = make_inputs("video_14b", heads=[0, 39])
    k = x["k"][0].float()
    norms = k.norm(dim=-1)  # [2, N]
    mask = torch.zeros(w.Nk, dtype=torch.bool)
    mask[idx] = True
    assert norms[:, mask].min() > 40  # x8 rows: |k| ~ 8 * sqrt(128) = 90
    assert norms[:, ~mask].max() < 20
    # the fp32 precision run draws the same values, unrounded
    f, _ = make_inputs("video_14b_fp32", Nq=2048, Nk=2048)
    g, _ = make_inputs("video_14b", Nq=2048, Nk=2048, heads=[0, 1])
    for t in TENSORS:
        assert f[t].dtype == torch.float32
        assert torch.equal(f[t].to(torch.bfloat16), g[t])


def test_head_shard_is_heads_of_the_full_draw():
    """One GPU's share of the 14B shape under an 8-way head split is heads 0-4
    of the 40-head draw, value for value."""
    w = WORKLOADS["video_14b_shard8"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d) == (1, 5, 32760, 32760, 128)
    a, s1 = make_inputs("video_14b_shard8", Nq=300, Nk=400)
    b, s2 = make_inputs("video_14b", Nq=300, Nk=400, heads=range(5))
    assert s1 == s2
    for t in TENSORS:
        assert torch.equal(a[t], b[t])


def test_unrounded_draws_round_to_the_bf16_draws():
    """dtype="fp32" gives the draws before their bf16 rounding: rounding them
    reproduces the bf16 workload exactly (no row-max step), or to within one
    bf16 rounding of the row scale (row-max step)."""
    for name in ("image_dit", "video_14b"):
        x, _ = make_inputs(name, Nq=40, Nk=50, heads=[1], device="cpu")
        y, _ = make_inputs(name, Nq=40, Nk=50, heads=[1], device="cpu", dtype="fp32")
        assert all(y[n].dtype == torch.float32 for n in y)
        for n in x:
            assert torch.equal(y[n].to(torch.bfloat16), x[n]), (name, n)
        assert any(not torch.equal(y[n], x[n].float()) for n in x)
    x, _ = make_inputs("video_1p3b", Nq=40, Nk=50, heads=[0], device="cpu")
    y, _ = make_inputs("video_1p3b", Nq=40, Nk=50, heads=[0], device="cpu", dtype="fp32")
    rel = ((y["q"] - x["q"].float()).abs() / x["q"].float().abs().clamp_min(1e-3)).max()
    assert rel < 2 ** -6  # two bf16 roundings and a row scale from rounded values
