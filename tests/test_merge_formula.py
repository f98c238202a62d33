"""The merge rule for partial results over disjoint key subsets, pinned on the
CPU against the fp64 oracle: the attention (and JVP) of all keys equals the
merge of the attentions of any partition of the keys.  This checks the formula
that attn_jvp_merge implements (the rule is stated in include/attn_jvp.h):

    lse = log sum_p exp(lse_p),  a_p = exp(lse_p - lse)
    O = sum_p a_p O_p,  mu = sum_p a_p mu_p,  dO = sum_p a_p (dO_p + mu_p O_p) - mu O

written here independently in NumPy.  The identity is exact up to rounding."""

import numpy as np
import pytest

import oracle


def merge(parts):
    lse_p = np.stack([p[2] for p in parts])
    m = lse_p.max(axis=0)
    w = np.exp(lse_p - m)
    a = w / w.sum(axis=0)
    lse = m + np.log(w.sum(axis=0))
    O = sum(a[i][..., None] * parts[i][0] for i in range(len(parts)))
    mu = sum(a[i] * parts[i][3] for i in range(len(parts)))
    H = sum(a[i][..., None] * (parts[i][1] + parts[i][3][..., None] * parts[i][0])
            for i in range(len(parts)))
    return O, H - mu[..., None] * O, lse, mu


@pytest.mark.parametrize("cuts", [[5], [1, 2], [10, 11, 30], [3, 4, 5, 6, 7, 20]])
def test_merge_of_key_partition_equals_whole(cuts):
    rng = np.random.default_rng(len(cuts))
    B, H, Nq, Nk, d = 1, 2, 9, 37, 8
    x = {n: rng.standard_normal((B, H, Nq if n in ("q", "dq") else Nk, d)) for n in
         ("q", "k", "v", "dq", "dk", "dv")}
    x["k"][:, :, 3] *= 6  # a dominant key in one part
    s = 0.7
    full = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], s, with_dlse=True)
    bounds = [0, *cuts, Nk]
    parts = []
    for j0, j1 in zip(bounds[:-1], bounds[1:]):
        sl = {n: (t if n in ("q", "dq") else t[:, :, j0:j1]) for n, t in x.items()}
        parts.append(oracle.attention_jvp(sl["q"], sl["k"], sl["v"], sl["dq"], sl["dk"], sl["dv"],
                                          s, with_dlse=True))
    got = merge(parts)
    for name, g, w in zip(("O", "dO", "lse", "dlse"), got, full):
        assert np.allclose(g, w, rtol=1e-12, atol=1e-12), name


def test_merge_rule_catches_a_dropped_term():
    """A planted mistake (dropping mu_p O_p from the merged sum) breaks the identity."""
    rng = np.random.default_rng(7)
    x = {n: rng.standard_normal((1, 1, 5 if n in ("q", "dq") else 12, 4)) for n in
         ("q", "k", "v", "dq", "dk", "dv")}
    full = oracle.attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], 0.5, with_dlse=True)
    parts = [oracle.attention_jvp(x["q"], x["k"][:, :, a:b], x["v"][:, :, a:b], x["dq"],
                                  x["dk"][:, :, a:b], x["dv"][:, :, a:b], 0.5, with_dlse=True)
             for a, b in ((0, 6), (6, 12))]
    assert np.allclose(merge(parts)[1], full[1], rtol=1e-12, atol=1e-12)
    O, dO, lse, mu = merge(parts)
    lse_p = np.stack([p[2] for p in parts])
    a = np.exp(lse_p - lse)
    dropped = sum(a[i][..., None] * parts[i][1] for i in range(2)) - mu[..., None] * O
    assert not np.allclose(dropped, full[1], rtol=1e-6, atol=1e-6)
