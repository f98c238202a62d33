"""Seeded synthetic inputs for the attention-JVP workloads.

This module is shared by the GPU tests, the benchmark and the oracle checks.
It only draws and shapes data; it holds none of attention's arithmetic (no
softmax, no output, no derivative).  Its one data-dependent step is the
logit-range placement of the 1.3B-video workload, which needs the largest dot
product max_j <q_i, k_j> of each query row (a float64 matmul followed by a max).

Shapes follow the video / image diffusion transformers that rCM distils
(Anthology of the SOTA record LIT-783, "Results (Tables 1-3)": Wan2.1 1.3B and
14B at 480p, Cosmos-Predict2 images; "JVP at production scale": self- and
cross-attention).  480p video for 5 s gives 21 x 30 x 52 = 32760 latent tokens.
All tensors are contiguous [B, H, N, d], tangents shaped like their primals.

Recipe (all seeded, reproducible on any host):

* Every (tensor, b, h) slice is drawn from its own ``torch.Generator`` seeded
  with ``seed*1000003 + tid*10007 + b*H + h`` (tid: q, k, v, dq, dk, dv = 0..5;
  H is the workload's full head count, so a subset of heads draws identical
  values), as float32 ``randn`` times sigma, then rounded to bf16 (RNE) for the
  bf16 workloads.
* ``row_max``: per (b, h) a generator seeded ``seed*1000003 + 7*10007 + b*H + h``
  draws t_i ~ U[lo, hi]; each query row is multiplied by t_i / m_i, where m_i is
  max_j scale * <q_i, k_j> over all keys in float64 from the bf16 values, and
  re-rounded to bf16.  The achieved row maxima are t_i up to bf16 rounding.
* ``outlier_frac``: for each of q, k, v a set of ceil(frac*N) token indices
  (``randperm`` seeded ``seed*1000003 + 6*10007 + tid``), shared by all heads
  and batches, is multiplied by ``outlier_scale`` (8 is exact in bf16);
  tangents are not scaled.
"""

import dataclasses
import math

import torch

TENSORS = ("q", "k", "v", "dq", "dk", "dv")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str                 # "bf16" or "fp32": the dtype of all six inputs
    sigma: tuple = (1.0, 1.0, 1.0, 0.1, 0.1, 0.1)   # std of q, k, v, dq, dk, dv
    row_max: tuple = None      # (lo, hi) for the per-row max logit, or None
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0
    seed_H: int = None         # head count used for seeding (default: H)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {w.name: w for w in [
    Workload("tiny_fp32", "fp32 self-attention JVP, B=1 H=2 N=256 d=64, all six inputs N(0,1)",
             1, 2, 256, 256, 64, "fp32", sigma=(1.0,) * 6),
    Workload("image_dit", "bf16 self-attention JVP shaped like an image DiT, B=2 H=16 N=4096 d=128",
             2, 16, 4096, 4096, 128, "bf16"),
    Workload("text_cross_frozen", "bf16 cross-attention JVP, 32760 video queries x 512 frozen text keys "
             "(dK = dV = 0), B=1 H=12 d=128", 1, 12, 32760, 512, 128, "bf16",
             sigma=(1.0, 1.0, 1.0, 0.1, 0.0, 0.0)),
    Workload("text_cross", "bf16 cross-attention JVP, 32760 video queries x 512 text keys with "
             "N(0, 0.1^2) key/value tangents, B=1 H=12 d=128", 1, 12, 32760, 512, 128, "bf16"),
    Workload("video_1p3b", "bf16 self-attention JVP shaped like a 1.3B video DiT, B=1 H=12 "
             "N=32760 (21x30x52 latents) d=128, per-row max logit in [5, 20]",
             1, 12, 32760, 32760, 128, "bf16", row_max=(5.0, 20.0)),
    Workload("video_14b", "bf16 self-attention JVP shaped like a 14B video DiT, B=1 H=40 N=32760 "
             "d=128, 1% of q/k/v token rows scaled x8", 1, 40, 32760, 32760, 128, "bf16",
             outlier_frac=0.01),
    Workload("video_14b_fp32", "fp32 run of the 14B video shape on its first 2 heads (unrounded "
             "draws, same outliers)", 1, 2, 32760, 32760, 128, "fp32",
             outlier_frac=0.01, seed_H=40),
    Workload("video_14b_shard8", "one GPU's share of the 14B video shape sharded by head over 8 "
             "GPUs: heads 0-4 of the 40-head draw, B=1 H=5 N=32760 d=128", 1, 5, 32760, 32760,
             128, "bf16", outlier_frac=0.01, seed_H=40),
]}


def _gen(seed):
    return torch.Generator().manual_seed(int(seed))


def slice_seed(seed, tid, b, h, H):
    return seed * 1000003 + tid * 10007 + b * H + h


def outlier_rows(seed, tid, N, frac):
    """The token indices scaled as outliers in tensor ``tid`` (0, 1, 2 = q, k, v)."""
    n = int(math.ceil(frac * N))
    return torch.randperm(N, generator=_gen(seed * 1000003 + 6 * 10007 + tid))[:n]


def _max_dot(q, k, device):
    """max_j <q_i, k_j> per row, float64 (a data statistic, computed in row chunks)."""
    dev = torch.device(device)
    kd = k.to(device=dev, dtype=torch.float64)
    out = torch.empty(q.shape[0], dtype=torch.float64)
    for r0 in range(0, q.shape[0], 4096):
        qd = q[r0:r0 + 4096].to(device=dev, dtype=torch.float64)
        out[r0:r0 + 4096] = (qd @ kd.T).amax(dim=1).cpu()
    return out


def make_inputs(name, seed=0, heads=None, Nq=None, Nk=None, device=None, dtype=None):
    """Draw the six input tensors of a workload on the CPU.

    ``heads`` restricts to a subset of head indices (same values as in the full
    draw); ``Nq``/``Nk`` override the sequence lengths with the same recipe
    (for reduced-size checks).  ``device`` is where the float64 max-dot-product
    of the ``row_max`` step runs (default: the GPU if one is visible).
    ``dtype="fp32"`` returns a bf16 workload's draws before they are rounded to
    bf16 (the row_max step then works on the fp32 values), for precision
    comparisons against unrounded inputs.
    Returns (dict of contiguous CPU tensors keyed by TENSORS, scale).
    """
    w = WORKLOADS[name]
    Nq = w.Nq if Nq is None else Nq
    Nk = w.Nk if Nk is None else Nk
    heads = list(range(w.H)) if heads is None else list(heads)
    H_seed = w.seed_H or w.H
    dtype = w.dtype if dtype is None else dtype
    if dtype not in ("bf16", "fp32"):
        raise ValueError("dtype must be 'bf16' or 'fp32'")
    out_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    lens = (Nq, Nk, Nk, Nq, Nk, Nk)
    outliers = {}
    if w.outlier_frac > 0:
        for tid in range(3):
            outliers[tid] = outlier_rows(seed, tid, lens[tid], w.outlier_frac)
    res = {t: torch.empty((w.B, len(heads), lens[i], w.d), dtype=out_dtype) for i, t in enumerate(TENSORS)}
    for b in range(w.B):
        for hi, h in enumerate(heads):
            for tid, t in enumerate(TENSORS):
                x = torch.randn(lens[tid], w.d, generator=_gen(slice_seed(seed, tid, b, h, H_seed)))
                x = x * w.sigma[tid]
                if tid in outliers:
                    x[outliers[tid]] *= w.outlier_scale
                res[t][b, hi] = x.to(out_dtype)
            if w.row_max is not None:
                lo, hi_ = w.row_max
                tgt = torch.empty(Nq, dtype=torch.float64).uniform_(
                    lo, hi_, generator=_gen(seed * 1000003 + 7 * 10007 + b * H_seed + h))
                m = w.scale * _max_dot(res["q"][b, hi], res["k"][b, hi], device)
                if bool((m <= 0).any()):
                    raise RuntimeError("row with a non-positive max logit; pick another seed")
                f = (tgt / m).to(torch.float32)
                res["q"][b, hi] = (res["q"][b, hi].to(torch.float32) * f[:, None]).to(out_dtype)
    return res, w.scale
