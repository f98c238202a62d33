"""Plain fp64 CPU oracle: softmax attention and its forward-mode derivative.

TEST INFRASTRUCTURE ONLY.  This module is the reference that the GPU path is
checked against.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it.  The product path
(the HIP library and its Python binding) never does, and it shares no code,
header, table or helper with it.

What it computes
----------------
The rCM record on the Anthology of the SOTA (LIT-783, "Key takeaways", the
"JVP at production scale (paper §3.2, App. C)" bullet) credits a kernel that
returns the FlashAttention-2 forward result and its directional derivative
along tangents of Q, K and V (shaped like Q, K and V) from a single fused
sweep, for keys from the queries' own sequence or from another one.  The pages
give no formula, so this oracle is the plain mathematical definition of that
result, not the tiled algorithm:

  per (batch, head), queries i < Nq, keys j < Nk, head dim d, scalar scale s

    S   = s * Q K^T                                   (Nq x Nk logits)
    P   = row-softmax(S)                              (two-pass: max, then exp/sum)
    O   = P V
    lse = m + ln(sum_j exp(S_ij - m)),  m = max_j S_ij   (natural log)

  and for a cotangent gO (the gradient of a loss with respect to O), the
  reverse-mode derivative (vector-Jacobian product) of the same map:

    gV  = P^T gO                                      (O = P V, in V)
    gP  = gO V^T                                      (O = P V, in P)
    gS  = P * (gP - D),  D_i = sum_j P_ij gP_ij       (adjoint of the softmax)
    gQ  = s gS K,  gK = s gS^T Q                      (S = s Q K^T)

  and for tangents dQ, dK, dV (a directional derivative of the map above):

    dS  = s * (dQ K^T + Q dK^T)                       (product rule on S)
    dP  = P * (dS - mu),  mu_i = sum_j P_ij dS_ij     (derivative of softmax)
    dO  = dP V + P dV                                 (product rule on P V)
    dlse = mu                                         (derivative of log-sum-exp)

Everything is float64.  There is no online softmax, no tiling over keys and no
fusion: rows are processed in chunks only to bound memory, which does not
change any value because rows are independent.

Parity pins: every function here is pinned in ``tests/test_oracle.py`` against
complex-step derivatives of a pure-Python brute-force attention, central finite
differences, closed forms, exact identities and ``torch.func.jvp``; nothing
here is "parity unpinned".
"""

import numpy as np

__all__ = ["attention", "attention_jvp", "attention_jvp_rows", "attention_vjp",
           "attention_vjp_keys"]

# Rows per chunk: bounds the Nq_chunk x Nk float64 temporaries (512 x 32760 x 8 B
# = 134 MB each) without changing any value.
ROW_CHUNK = 512


def _f64(x):
    """Exact upcast to float64 (bf16 and fp32 values are exactly representable)."""
    if hasattr(x, "detach"):  # a torch tensor: go through torch's exact upcast
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _head_forward(q, k, v, scale):
    """Softmax attention for one head: q [n, d], k and v [Nk, d] -> (O, lse, P).

    The definition: S = s Q K^T, P = softmax over keys, O = P V.
    """
    S = scale * (q @ k.T)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    O = P @ v
    lse = m[:, 0] + np.log(l[:, 0])
    return O, lse, P


def _head_jvp(q, k, v, dq, dk, dv, scale):
    """Attention and its JVP for one head and a chunk of query rows.

    Returns (O, dO, lse, dlse).  Each line is one rule of calculus applied to
    the forward definition in ``_head_forward``.
    """
    O, lse, P = _head_forward(q, k, v, scale)
    # S = s q k^T is bilinear in (q, k): its derivative is s (dq k^T + q dk^T).
    dS = scale * (dq @ k.T + q @ dk.T)
    # softmax'(S)[dS] = P * (dS - <P, dS>_row); the row mean-shift is mu.
    mu = (P * dS).sum(axis=1)
    dP = P * (dS - mu[:, None])
    # O = P v is bilinear in (P, v): dO = dP v + P dv.
    dO = dP @ v + P @ dv
    # lse = log sum exp(S): its derivative is sum_j P_ij dS_ij = mu.
    return O, dO, lse, mu


def _head_vjp(q, k, v, go, scale):
    """Gradients of <gO, O> for one head: q [n, d], k and v [Nk, d], go [n, d].

    Each line is the adjoint of one line of ``_head_forward``."""
    _, _, P = _head_forward(q, k, v, scale)
    gV = P.T @ go
    gP = go @ v.T
    D = (P * gP).sum(axis=1, keepdims=True)
    gS = P * (gP - D)
    return scale * (gS @ k), scale * (gS.T @ q), gV


def attention_vjp(q, k, v, go, scale):
    """Reverse-mode derivative: the gradients (gQ, gK, gV) of sum(gO * O) with
    respect to Q, K and V.  q, go: [B, H, Nq, d]; k, v: [B, H, Nk, d].  Float64.

    Query rows are processed in chunks (memory only): gQ is per row, and the
    key-side gradients gK, gV are sums over rows, accumulated chunk by chunk.
    """
    q, k, v, go = (_f64(t) for t in (q, k, v, go))
    B, H, Nq, d = q.shape
    gq = np.empty_like(q)
    gk = np.zeros_like(k)
    gv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, ROW_CHUNK):
                r1 = min(Nq, r0 + ROW_CHUNK)
                a, c, e = _head_vjp(q[b, h, r0:r1], k[b, h], v[b, h], go[b, h, r0:r1], scale)
                gq[b, h, r0:r1] = a
                gk[b, h] += c
                gv[b, h] += e
    return gq, gk, gv


def attention_vjp_keys(q, k, v, go, scale, b, h, keys):
    """gK and gV of ``attention_vjp`` for selected key rows of one (b, h) head.

    A key's gradients sum over every query: gK_j = s sum_i gS_ij q_i and
    gV_j = sum_i P_ij gO_i, where P_ij and gS_ij need the whole row i (its
    softmax normaliser and D_i = sum_j' P_ij' gP_ij').  So every query row is
    still processed, in chunks, with all keys for P and D, and only the
    selected key columns are kept for the sums.  Returns (gK, gV) for ``keys``
    (an int array), float64.
    """
    keys = np.asarray(keys, dtype=np.int64)
    qb, kb, vb, gob = (_f64(t[b, h]) for t in (q, k, v, go))
    gk = np.zeros((len(keys), kb.shape[-1]))
    gv = np.zeros((len(keys), vb.shape[-1]))
    for r0 in range(0, qb.shape[0], ROW_CHUNK):
        r1 = min(qb.shape[0], r0 + ROW_CHUNK)
        _, _, P = _head_forward(qb[r0:r1], kb, vb, scale)
        gP = gob[r0:r1] @ vb.T
        D = (P * gP).sum(axis=1, keepdims=True)
        gS = P[:, keys] * (gP[:, keys] - D)
        gk += scale * (gS.T @ qb[r0:r1])
        gv += P[:, keys].T @ gob[r0:r1]
    return gk, gv


def attention(q, k, v, scale):
    """Forward only.  q [B, H, Nq, d]; k, v [B, H, Nk, d].  Returns (O, lse) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    O = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, ROW_CHUNK):
                r1 = min(Nq, r0 + ROW_CHUNK)
                o, l_, _ = _head_forward(q[b, h, r0:r1], k[b, h], v[b, h], scale)
                O[b, h, r0:r1] = o
                lse[b, h, r0:r1] = l_
    return O, lse


def attention_jvp(q, k, v, dq, dk, dv, scale, with_dlse=False):
    """Attention and its JVP over whole tensors.

    q, dq: [B, H, Nq, d]; k, v, dk, dv: [B, H, Nk, d] (numpy or torch, any float
    dtype; upcast exactly to float64).  Returns (O, dO, lse) as float64 numpy
    arrays of shapes [B, H, Nq, d], [B, H, Nq, d], [B, H, Nq]; with
    ``with_dlse`` also the tangent of lse, [B, H, Nq].
    """
    q, k, v, dq, dk, dv = (_f64(t) for t in (q, k, v, dq, dk, dv))
    B, H, Nq, d = q.shape
    O = np.empty((B, H, Nq, v.shape[-1]))
    dO = np.empty_like(O)
    lse = np.empty((B, H, Nq))
    dlse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, ROW_CHUNK):
                r1 = min(Nq, r0 + ROW_CHUNK)
                o, do, l_, dl = _head_jvp(q[b, h, r0:r1], k[b, h], v[b, h],
                                          dq[b, h, r0:r1], dk[b, h], dv[b, h], scale)
                O[b, h, r0:r1], dO[b, h, r0:r1] = o, do
                lse[b, h, r0:r1], dlse[b, h, r0:r1] = l_, dl
    if with_dlse:
        return O, dO, lse, dlse
    return O, dO, lse


def attention_jvp_rows(q, k, v, dq, dk, dv, scale, b, h, rows):
    """Attention and JVP for selected query rows of one (b, h) head.

    Rows are independent, so this equals the corresponding rows of
    ``attention_jvp``; it lets full-size tensors be checked on a sample.
    Returns (O, dO, lse) for ``rows`` (an int array), float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qb, dqb = _f64(q[b, h][rows]), _f64(dq[b, h][rows])
    kb, vb, dkb, dvb = _f64(k[b, h]), _f64(v[b, h]), _f64(dk[b, h]), _f64(dv[b, h])
    O = np.empty((len(rows), vb.shape[-1]))
    dO = np.empty_like(O)
    lse = np.empty(len(rows))
    for r0 in range(0, len(rows), ROW_CHUNK):
        r1 = min(len(rows), r0 + ROW_CHUNK)
        o, do, l_, _ = _head_jvp(qb[r0:r1], kb, vb, dqb[r0:r1], dkb, dvb, scale)
        O[r0:r1], dO[r0:r1], lse[r0:r1] = o, do, l_
    return O, dO, lse
