"""Shared helpers for the GPU parity tests (not collected by pytest).

Inputs come from ``workloads`` (seeded, on the CPU); the same CPU tensors feed
the fp64 oracle and, copied to the device, the HIP library through its C ABI.
"""

import numpy as np
import torch

import attention_forward_mode_amd as ajvp
import oracle

NAMES = ("q", "k", "v", "dq", "dk", "dv")

# bf16 gate (max-abs and relative Frobenius on O, dO and lse)
BF16_MAX_ABS = 2e-2
BF16_REL_FROB = 1e-2
# fp32 gate
F32_REL_FROB = 1e-5


def to_device(x, dev="cuda:0"):
    return {n: x[n].to(dev) for n in NAMES}


def run(g, scale, lse=True):
    args = [g[n] for n in NAMES]
    # name the case before the launch, so a device fault can be traced to it
    print(f"  launch {str(g['q'].dtype)[6:]} q{tuple(g['q'].shape)} k{tuple(g['k'].shape)} "
          f"scale={scale:.4g}", flush=True)
    if g["q"].dtype == torch.bfloat16:
        out = ajvp.attn_jvp_fwd(*args, scale=scale, lse=lse)
    else:
        out = ajvp.attn_jvp_fwd_f32(*args, scale=scale, lse=lse)
    torch.cuda.synchronize()
    return out


def metrics(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    return {
        "max_abs": float(err.max()),
        "rel_frob": float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)),
        "max_rel": float(err.max() / max(np.abs(want).max(), 1e-300)),
    }


def check(label, outs, refs, fp32):
    """Assert the gate on (O, dO, lse) and print the figures."""
    for name, got, want in zip(("O", "dO", "lse"), outs, refs):
        if got is None:
            continue
        if isinstance(got, torch.Tensor):
            got = got.double().cpu().numpy()
        m = metrics(got, want)
        print(f"[{label}] {name}: max-abs {m['max_abs']:.3e} rel-Frobenius {m['rel_frob']:.3e} "
              f"max-abs/max|ref| {m['max_rel']:.3e}", flush=True)
        assert np.isfinite(got).all(), f"{label} {name}: non-finite output"
        if fp32:
            assert m["rel_frob"] <= F32_REL_FROB, (label, name, m)
        else:
            assert m["max_abs"] <= BF16_MAX_ABS and m["rel_frob"] <= BF16_REL_FROB, (label, name, m)


def sample_rows(Nq, n, rng, extra=()):
    """n random query rows plus the first and last rows (the ragged tail) and extras."""
    rows = set(rng.choice(Nq, size=min(n, Nq), replace=False).tolist())
    rows |= {0, Nq - 1, max(0, Nq - 128)}
    rows |= {int(r) for r in extra if 0 <= int(r) < Nq}
    return np.array(sorted(rows), dtype=np.int64)


def check_sampled(label, x, scale, outs, rows_per_head=24, seed=0, extra_rows=()):
    """Compare full-size outputs with the oracle on sampled rows of every (b, h)."""
    o, to, lse = (t.cpu() if t is not None else None for t in outs)
    B, H, Nq, _ = x["q"].shape
    rng = np.random.default_rng(seed)
    got_o, got_do, got_l, ref_o, ref_do, ref_l = [], [], [], [], [], []
    for b in range(B):
        for h in range(H):
            rows = sample_rows(Nq, rows_per_head, rng, extra_rows)
            O, dO, L = oracle.attention_jvp_rows(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                                 scale, b, h, rows)
            ref_o.append(O), ref_do.append(dO), ref_l.append(L)
            got_o.append(o[b, h, rows].double().numpy())
            got_do.append(to[b, h, rows].double().numpy())
            if lse is not None:
                got_l.append(lse[b, h, rows].double().numpy())
    outs_s = (np.concatenate(got_o), np.concatenate(got_do),
              np.concatenate(got_l) if got_l else None)
    refs_s = (np.concatenate(ref_o), np.concatenate(ref_do), np.concatenate(ref_l))
    check(label, outs_s, refs_s, fp32=x["q"].dtype == torch.float32)
    # properties of every row, at full size
    for t, name in ((o, "O"), (to, "dO"), (lse, "lse")):
        if t is not None:
            assert torch.isfinite(t).all(), f"{label}: non-finite {name} somewhere"
    # O is a convex combination of the rows of V: every column stays in V's range
    vmin = x["v"].float().amin(dim=2, keepdim=True)
    vmax = x["v"].float().amax(dim=2, keepdim=True)
    slack = 1e-2 * x["v"].float().abs().amax()
    assert bool(((o >= vmin - slack) & (o <= vmax + slack)).all()), f"{label}: O outside V's hull"
