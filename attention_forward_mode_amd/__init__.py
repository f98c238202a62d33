"""Python binding of libattn_jvp.so: fused attention forward + JVP on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn_jvp.h``; torch supplies
device memory and the current stream.  The names mirror the C entry points:

    attn_jvp_fwd(q, k, v, tq, tk, tv, scale=None, lse=True) -> (o, to, lse)
        bf16 inputs [B, H, Nq|Nk, d] on the GPU; fp32 outputs
    attn_jvp_pack_kv(k, v, tk, tv, workspace=None) -> workspace
    attn_jvp_fwd_packed(q, tq, workspace, Nk, ...) -> (o, to, lse)
        the two phases of attn_jvp_fwd, callable separately
    attn_jvp_fwd_ex(q, k, v, tq=None, tk=None, tv=None, ...) -> (o, to, lse, tlse)
        NULL (None) tangents, the tangent of lse, fp32 or bf16 outputs
    attn_fwd(q, k, v, ...) -> (o, lse)    forward attention alone
    attn_jvp_merge(lse_parts, o_parts, to_parts=None, tlse_parts=None)
        -> (lse, o, to, tlse): combine results over disjoint key subsets
    attn_bwd(q, k, v, o, go, lse) -> (gq, gk, gv)
        the backward pass: gradients of a loss through O
    attn_jvp_fwd_noalloc(q, k, v, tq, tk, tv, ...) -> (o, to, lse)
        attn_jvp_fwd without any allocation in the library (its tile images in
        a fixed device buffer of NOALLOC_BYTES per GPU)
    attn_jvp_fwd_f32(...)  the same with fp32 inputs
    attn_jvp_workspace_bytes(B, H, Nk, d)
    attn_jvp_strerror(status)

The operation (rCM record LIT-783, Anthology of the SOTA, "Key takeaways",
"JVP at production scale", paper §3.2 / App. C): O = softmax(s Q K^T) V, its
tangent dO along (dQ, dK, dV), and lse = ln sum_j exp(s q_i . k_j).

If the shared library has not been built, the first call raises ImportError:
there is no fallback implementation.
"""

import ctypes
import math
import os

import torch

__all__ = ["attn_jvp_fwd", "attn_jvp_fwd_noalloc", "NOALLOC_BYTES", "attn_jvp_pack_kv", "attn_jvp_fwd_packed", "attn_jvp_fwd_ex", "attn_fwd",
           "attn_jvp_merge", "attn_bwd", "attn_bwd_workspace_bytes", "attn_jvp_fwd_f32",
           "attn_jvp_workspace_bytes",
           "attn_jvp_strerror", "AttnJvpError", "LIB_PATH", "lib"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_jvp.so")

_lib = None


def lib():
    """The loaded shared library (loaded on first use).

    Raises ImportError if it has not been built: there is no fallback.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m attention_forward_mode_amd.build "
            "or __graft_entry__.build()); there is no non-HIP fallback")
    L = ctypes.CDLL(LIB_PATH)
    _vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_jvp_fwd.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _vp]
    L.attn_jvp_fwd.restype = _i
    L.attn_jvp_fwd_noalloc.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _vp]
    L.attn_jvp_fwd_noalloc.restype = _i
    L.attn_jvp_fwd_ws.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _vp, _sz, _vp]
    L.attn_jvp_fwd_ws.restype = _i
    L.attn_jvp_pack_kv.argtypes = [_vp] * 4 + [_i] * 4 + [_vp, _sz, _vp]
    L.attn_jvp_pack_kv.restype = _i
    L.attn_jvp_fwd_packed.argtypes = [_vp] * 3 + [_sz] + [_vp] * 3 + [_i] * 5 + [_f, _vp]
    L.attn_jvp_fwd_packed.restype = _i
    L.attn_jvp_fwd_ex.argtypes = [_vp] * 10 + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
    L.attn_jvp_fwd_ex.restype = _i
    L.attn_jvp_fwd_splitkv.argtypes = [_vp] * 10 + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
    L.attn_jvp_fwd_splitkv.restype = _i
    L.attn_jvp_splitkv_workspace_bytes.argtypes = [_i] * 6
    L.attn_jvp_splitkv_workspace_bytes.restype = _sz
    L.attn_fwd_splitkv.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
    L.attn_fwd_splitkv.restype = _i
    L.attn_fwd.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _vp, _sz, _vp]
    L.attn_fwd.restype = _i
    L.attn_jvp_merge.argtypes = [_vp] * 4 + [_i] * 3 + [_vp] * 5
    L.attn_jvp_merge.restype = _i
    L.attn_bwd.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _vp, _sz, _vp]
    L.attn_bwd.restype = _i
    L.attn_bwd_workspace_bytes.argtypes = [_i] * 5
    L.attn_bwd_workspace_bytes.restype = _sz
    L.attn_jvp_fwd_f32.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _vp]
    L.attn_jvp_fwd_f32.restype = _i
    L.attn_jvp_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.attn_jvp_workspace_bytes.restype = _sz
    L.attn_jvp_strerror.argtypes = [_i]
    L.attn_jvp_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


OK, EINVAL, EUNSUPPORTED, EALIGN, ELAUNCH = 0, -1, -2, -3, -4
NOALLOC_BYTES = 128 << 20  # the device buffer of attn_jvp_fwd_noalloc (ATTN_JVP_NOALLOC_BYTES)
OUT_F32, OUT_BF16 = 0, 1


class AttnJvpError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"attn_jvp: {attn_jvp_strerror(status)} (status {status})")


def attn_jvp_strerror(status):
    return lib().attn_jvp_strerror(int(status)).decode()


def attn_jvp_workspace_bytes(B, H, Nk, d):
    return int(lib().attn_jvp_workspace_bytes(B, H, Nk, d))


def _check(q, k, v, tq, tk, tv, dtype):
    for name, t in (("q", q), ("k", k), ("v", v), ("tq", tq), ("tk", tk), ("tv", tv)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tq.shape != q.shape:
        raise ValueError("tq must have q's shape")
    for name, t in (("k", k), ("v", v), ("tk", tk), ("tv", tv)):
        if t.shape != (B, H, Nk, d):
            raise ValueError(f"{name} must be {(B, H, Nk, d)}, got {tuple(t.shape)}")
    dev = q.device
    if any(t.device != dev for t in (k, v, tq, tk, tv)):
        raise ValueError("all inputs must be on one device")
    return B, H, Nq, Nk, d


def _outputs(q, B, H, Nq, d, want_lse, out):
    if out is not None:
        o, to, lse = out
        for name, t, shape in (("o", o, (B, H, Nq, d)), ("to", to, (B, H, Nq, d)),
                               ("lse", lse, (B, H, Nq))):
            if t is None and name == "lse":
                continue
            if (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()
                    or t.device != q.device):
                raise ValueError(f"out {name} must be a contiguous fp32 {shape} tensor on {q.device}")
    else:
        o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
        to = torch.empty_like(o)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    return o, to, lse


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _workspace(ws, B, H, Nk, d, device):
    """The caller's workspace (checked) or a new one from torch's caching allocator."""
    if ws is None:
        return torch.empty(max(attn_jvp_workspace_bytes(B, H, Nk, d), 1), dtype=torch.uint8,
                           device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws


def _nbytes(t):
    return t.numel() * t.element_size()


def attn_jvp_pack_kv(k, v, tk, tv, workspace=None):
    """Phase 1 of the bf16 path: pack K, V, dK, dV ([B, H, Nk, d] bf16) into
    the tile images the fused kernel copies into LDS.  Returns the workspace (a
    new uint8 tensor unless one is passed).  Launches on the current stream."""
    for name, t in (("k", k), ("v", v), ("tk", tk), ("tv", tv)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda
                or t.dim() != 4 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous 4-D bf16 GPU tensor")
    for name, t in (("v", v), ("tk", tk), ("tv", tv)):
        if t.shape != k.shape or t.device != k.device:
            raise ValueError(f"{name} must have k's shape and device")
    B, H, Nk, d = k.shape
    workspace = _workspace(workspace, B, H, Nk, d, k.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(k.device).cuda_stream)
    with torch.cuda.device(k.device):
        rc = lib().attn_jvp_pack_kv(_ptr(k), _ptr(v), _ptr(tk), _ptr(tv), B, H, Nk, d,
                                    _ptr(workspace), _nbytes(workspace), stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return workspace


def attn_jvp_fwd_packed(q, tq, workspace, Nk, scale=None, lse=True, out=None):
    """Phase 2 of the bf16 path: attention + JVP from q, tq and a workspace
    filled by ``attn_jvp_pack_kv`` for Nk keys of the same B, H, d.  Returns
    (o, to, lse) like ``attn_jvp_fwd``."""
    B, H, Nq, _, d = _check(q, q, q, tq, q, q, torch.bfloat16)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if workspace is None:
        raise ValueError("workspace must come from attn_jvp_pack_kv")
    workspace = _workspace(workspace, B, H, Nk, d, q.device)
    o, to, lse_t = _outputs(q, B, H, Nq, d, lse, out)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_packed(_ptr(q), _ptr(tq), _ptr(workspace), _nbytes(workspace),
                                       _ptr(o), _ptr(to), _ptr(lse_t), B, H, Nq, int(Nk), d, s,
                                       stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t


def attn_jvp_fwd(q, k, v, tq, tk, tv, scale=None, lse=True, out=None, workspace=None):
    """bf16 attention + JVP.  Returns (o, to, lse) fp32 (lse None if lse=False).

    ``out`` may pass preallocated (o, to, lse) fp32 tensors; ``workspace`` a
    uint8 device tensor of at least ``attn_jvp_workspace_bytes`` bytes (by
    default one is taken from torch's caching allocator).  Launches on the
    current stream; does not synchronise.
    """
    B, H, Nq, Nk, d = _check(q, k, v, tq, tk, tv, torch.bfloat16)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, to, lse_t = _outputs(q, B, H, Nq, d, lse, out)
    workspace = _workspace(workspace, B, H, Nk, d, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                 _ptr(o), _ptr(to), _ptr(lse_t), B, H, Nq, Nk, d, s,
                                 _ptr(workspace), _nbytes(workspace), stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t


def attn_jvp_fwd_noalloc(q, k, v, tq, tk, tv, scale=None, lse=True, out=None):
    """attn_jvp_fwd through the entry point that allocates nothing: the library
    keeps the tile images in its fixed device buffer (calls that overlap on one
    GPU race on it).  ``out`` may pass preallocated (o, to, lse); otherwise torch
    allocates the outputs here, in the binding.  Returns (o, to, lse)."""
    B, H, Nq, Nk, d = _check(q, k, v, tq, tk, tv, torch.bfloat16)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, to, lse_t = _outputs(q, B, H, Nq, d, lse, out)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                        _ptr(o), _ptr(to), _ptr(lse_t), B, H, Nq, Nk, d, s,
                                        stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t


def _out_code(out_dtype):
    if out_dtype == torch.float32:
        return OUT_F32
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")


def _check_opt(t, like, name):
    """An optional tangent: None, or a tensor exactly like its primal."""
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or t.dtype != like.dtype or t.shape != like.shape
            or t.device != like.device or not t.is_contiguous()):
        raise ValueError(f"{name} must be None or a contiguous tensor like its primal")


def _ws_arg(workspace, device):
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return _ptr(workspace), _nbytes(workspace)


def attn_jvp_fwd_ex(q, k, v, tq=None, tk=None, tv=None, scale=None, lse=True, tlse=True,
                    out_dtype=torch.float32, workspace=None):
    """bf16 attention + JVP with optional tangents (None = zero; tk = tv = None
    runs the frozen-key kernel), the tangent of lse, and fp32 or bf16 outputs.
    Returns (o, to, lse, tlse); lse / tlse are None when not requested.  With
    workspace=None the library's stream-ordered pool provides it."""
    B, H, Nq, Nk, d = _check(q, k, v, q, k, v, torch.bfloat16)
    _check_opt(tq, q, "tq")
    _check_opt(tk, k, "tk")
    _check_opt(tv, v, "tv")
    code = _out_code(out_dtype)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    to = torch.empty_like(o)
    lse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse else None
    tlse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if tlse else None
    wp, wb = _ws_arg(workspace, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                   _ptr(o), _ptr(to), _ptr(lse_t), _ptr(tlse_t), B, H, Nq, Nk, d,
                                   s, code, wp, wb, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t, tlse_t


def attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit=0):
    return int(lib().attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit))


def attn_jvp_fwd_splitkv(q, k, v, tq=None, tk=None, tv=None, scale=None, nsplit=0, lse=True,
                         tlse=True, workspace=None):
    """attn_jvp_fwd_ex with the key tiles cut into nsplit ranges (0: chosen
    from the sizes) on separate workgroups and the partial states merged: for
    few query rows against many keys.  fp32 outputs; returns (o, to, lse, tlse)."""
    B, H, Nq, Nk, d = _check(q, k, v, q, k, v, torch.bfloat16)
    _check_opt(tq, q, "tq")
    _check_opt(tk, k, "tk")
    _check_opt(tv, v, "tv")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    to = torch.empty_like(o)
    lse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse else None
    tlse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if tlse else None
    wp, wb = _ws_arg(workspace, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                        _ptr(o), _ptr(to), _ptr(lse_t), _ptr(tlse_t), B, H, Nq,
                                        Nk, d, s, int(nsplit), wp, wb, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t, tlse_t


def attn_fwd_splitkv(q, k, v, scale=None, nsplit=0, lse=True, workspace=None):
    """attn_fwd with the key tiles cut into nsplit ranges (0: chosen from the
    sizes) and the partial states merged.  fp32 outputs; returns (o, lse)."""
    B, H, Nq, Nk, d = _check(q, k, v, q, k, v, torch.bfloat16)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    lse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse else None
    wp, wb = _ws_arg(workspace, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Nq, Nk,
                                    d, s, int(nsplit), wp, wb, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, lse_t


def attn_fwd(q, k, v, scale=None, lse=True, out_dtype=torch.float32, workspace=None):
    """Forward attention alone (bf16 inputs): returns (o, lse)."""
    B, H, Nq, Nk, d = _check(q, k, v, q, k, v, torch.bfloat16)
    code = _out_code(out_dtype)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    lse_t = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse else None
    wp, wb = _ws_arg(workspace, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Nq, Nk, d, s,
                            code, wp, wb, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, lse_t


def attn_jvp_merge(lse_parts, o_parts, to_parts=None, tlse_parts=None):
    """Merge P partial results over disjoint key subsets.  lse_parts [P, *rows],
    o_parts [P, *rows, d] (fp32, contiguous, on the GPU), to_parts / tlse_parts
    like them or both None.  Returns (lse, o, to, tlse) with the part axis
    removed (to, tlse None for a forward-only merge)."""
    for name, t in (("lse_parts", lse_parts), ("o_parts", o_parts), ("to_parts", to_parts),
                    ("tlse_parts", tlse_parts)):
        if t is None and name in ("to_parts", "tlse_parts"):
            continue
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
    if (to_parts is None) != (tlse_parts is None):
        raise ValueError("to_parts and tlse_parts go together")
    P = lse_parts.shape[0]
    rows = tuple(lse_parts.shape[1:])
    d = o_parts.shape[-1]
    if tuple(o_parts.shape) != (P, *rows, d):
        raise ValueError("o_parts must be [P, *rows, d] matching lse_parts")
    if to_parts is not None and (to_parts.shape != o_parts.shape or tlse_parts.shape != lse_parts.shape):
        raise ValueError("to_parts / tlse_parts must match o_parts / lse_parts")
    R = int(math.prod(rows))
    dev = lse_parts.device
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    o = torch.empty((*rows, d), dtype=torch.float32, device=dev)
    to = torch.empty_like(o) if to_parts is not None else None
    tlse = torch.empty_like(lse) if to_parts is not None else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    with torch.cuda.device(dev):
        rc = lib().attn_jvp_merge(_ptr(lse_parts), _ptr(o_parts), _ptr(to_parts), _ptr(tlse_parts),
                                  P, R, d, _ptr(lse), _ptr(o), _ptr(to), _ptr(tlse), stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return lse, o, to, tlse


def attn_bwd_workspace_bytes(B, H, Nq, Nk, d):
    return int(lib().attn_bwd_workspace_bytes(B, H, Nq, Nk, d))


def attn_bwd(q, k, v, o, go, lse, scale=None, workspace=None):
    """Backward pass: gradients (gq, gk, gv) (fp32) of a loss through O, from
    bf16 q, k, v, the cotangent go (bf16, like q) and the forward's fp32 o
    and lse.  Launches on the current stream."""
    B, H, Nq, Nk, d = _check(q, k, v, go, k, v, torch.bfloat16)
    if (not isinstance(o, torch.Tensor) or o.dtype != torch.float32 or tuple(o.shape) != (B, H, Nq, d)
            or not o.is_contiguous() or o.device != q.device):
        raise ValueError("o must be the forward's contiguous fp32 [B, H, Nq, d] output")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be the forward's contiguous fp32 [B, H, Nq] lse")
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    gq = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    gk = torch.empty((B, H, Nk, d), dtype=torch.float32, device=q.device)
    gv = torch.empty_like(gk)
    wp, wb = _ws_arg(workspace, q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(go), _ptr(lse), _ptr(gq),
                            _ptr(gk), _ptr(gv), B, H, Nq, Nk, d, s, wp, wb, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return gq, gk, gv


def attn_jvp_fwd_f32(q, k, v, tq, tk, tv, scale=None, lse=True, out=None):
    """fp32 attention + JVP.  Returns (o, to, lse) fp32 (lse None if lse=False)."""
    B, H, Nq, Nk, d = _check(q, k, v, tq, tk, tv, torch.float32)
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o, to, lse_t = _outputs(q, B, H, Nq, d, lse, out)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    with torch.cuda.device(q.device):
        rc = lib().attn_jvp_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv),
                                  _ptr(o), _ptr(to), _ptr(lse_t), B, H, Nq, Nk, d, s, stream)
    if rc != OK:
        raise AttnJvpError(rc)
    return o, to, lse_t
