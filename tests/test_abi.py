"""The C ABI boundary, checked without a GPU: the library loads, exports every
entry point declared in include/*.h, and rejects bad arguments before it
launches anything (so no device is touched)."""

import ctypes
import glob
import os
import re

import pytest

import attention_forward_mode_amd as ajvp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, EINVAL, EUNSUPPORTED, EALIGN, ELAUNCH = 0, -1, -2, -3, -4


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        # declarations start a line: "ATTN_JVP_API <type> name(" (skip the macro's definition)
        names += re.findall(r"^ATTN_JVP_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return names


def test_library_loads_and_exports_every_declared_symbol():
    L = ajvp.lib()
    names = declared_functions()
    assert set(names) >= {"attn_jvp_fwd", "attn_jvp_fwd_ws", "attn_jvp_fwd_f32",
                          "attn_jvp_workspace_bytes", "attn_jvp_strerror"}
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def test_error_codes_match_header():
    text = open(os.path.join(ROOT, "include", "attn_jvp.h")).read()
    codes = dict(re.findall(r"#define (ATTN_JVP_\w+) \(?(-?\d+)\)?", text))
    outs = {k: int(codes.pop(k)) for k in list(codes) if k.startswith("ATTN_JVP_OUT_")}
    assert outs == {"ATTN_JVP_OUT_F32": ajvp.OUT_F32, "ATTN_JVP_OUT_BF16": ajvp.OUT_BF16}
    assert {k: int(v) for k, v in codes.items()} == {
        "ATTN_JVP_OK": OK, "ATTN_JVP_EINVAL": EINVAL, "ATTN_JVP_EUNSUPPORTED": EUNSUPPORTED,
        "ATTN_JVP_EALIGN": EALIGN, "ATTN_JVP_ELAUNCH": ELAUNCH}


def test_strerror():
    for code in (OK, EINVAL, EUNSUPPORTED, EALIGN, ELAUNCH, 12345):
        msg = ajvp.attn_jvp_strerror(code)
        assert isinstance(msg, str) and msg
    assert ajvp.attn_jvp_strerror(OK) == "ok"
    assert ajvp.attn_jvp_strerror(12345) == "unknown status"


def test_workspace_bytes():
    # per (b, h): one tile image per 64-key tile (K, dK as 64 x d bf16 and V^T,
    # dV^T as d x 64 fp16, unpadded operand fragments, a whole number of
    # 8 KiB), then a 2 KiB header (the fp16 exponents, the range pass's
    # partial maxima and the largest key norms)
    def img(d):
        used = 2 * 64 * d * 2 + 2 * d * 64 * 2
        return -(-used // 8192) * 8192
    hdr = 2048
    assert img(128) == 64 * 1024 and img(64) == 32 * 1024
    assert ajvp.attn_jvp_workspace_bytes(1, 1, 1, 128) == img(128) + hdr
    assert ajvp.attn_jvp_workspace_bytes(1, 12, 32760, 128) == 12 * (512 * img(128) + hdr)
    assert ajvp.attn_jvp_workspace_bytes(2, 3, 65, 64) == 6 * (2 * img(64) + hdr)
    assert ajvp.attn_jvp_workspace_bytes(0, 1, 1, 128) == 0
    assert ajvp.attn_jvp_workspace_bytes(1, 1, 1, 96) == 0


# Fake, never-dereferenced device addresses: every call below must be rejected
# by validation before any launch.
A = 0x7F0000000000  # 256-byte aligned


def _call(fn, ptrs=None, B=1, H=1, Nq=4, Nk=4, d=128, scale=0.1, ws=None, ws_bytes=None):
    L = ajvp.lib()
    p = [A + i * 0x100000 for i in range(9)] if ptrs is None else ptrs
    args = [ctypes.c_void_p(x) for x in p] + [B, H, Nq, Nk, d, ctypes.c_float(scale)]
    if fn == "attn_jvp_fwd_ws":
        nb = ajvp.attn_jvp_workspace_bytes(max(B, 1), max(H, 1), max(Nk, 1), d)
        args += [ctypes.c_void_p(A + 0x1000000 if ws is None else ws),
                 ctypes.c_size_t(nb if ws_bytes is None else ws_bytes)]
    args.append(ctypes.c_void_p(0))
    return getattr(L, fn)(*args)


def test_mfma_probe_library():
    """The matrix-core probe beside the library (include/mfma_probe.h, timed by
    bench.py) loads, exports its one entry point and rejects bad arguments
    before launching."""
    L = ctypes.CDLL(os.path.join(ROOT, "attention_forward_mode_amd", "libmfma_probe.so"))
    f = L.mfma_probe_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(1, 1, None, None) == -1
    assert f(0, 1, ctypes.c_void_p(A), None) == -1
    assert f(1, 0, ctypes.c_void_p(A), None) == -1


FNS = ["attn_jvp_fwd", "attn_jvp_fwd_ws", "attn_jvp_fwd_f32"]


@pytest.mark.parametrize("fn", FNS)
def test_null_pointers(fn):
    for i in range(8):  # q k v tq tk tv o to (lse may be NULL)
        p = [A + j * 0x100000 for j in range(9)]
        p[i] = 0
        assert _call(fn, p) == EINVAL, i


@pytest.mark.parametrize("fn", FNS)
def test_bad_sizes(fn):
    for kw in (dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0), dict(B=-1), dict(Nq=-5)):
        assert _call(fn, **kw) == EINVAL, kw


@pytest.mark.parametrize("fn", FNS)
def test_bad_scale(fn):
    # any finite scale is valid (a negative one too); NaN and +-Inf are not
    for s in (float("nan"), float("inf"), -float("inf")):
        assert _call(fn, scale=s) == EINVAL, s


@pytest.mark.parametrize("fn", FNS)
def test_unsupported_head_dim(fn):
    for d in (0, 32, 96, 256):
        rc = _call(fn, d=d)
        assert rc in (EUNSUPPORTED, EINVAL), (d, rc)
    assert _call(fn, d=96) == EUNSUPPORTED


@pytest.mark.parametrize("fn", FNS)
def test_oversized_slice(fn):
    # one slice of K past 2^31 bytes: outside what 32-bit buffer offsets reach
    assert _call(fn, Nk=1 << 24) == EUNSUPPORTED
    # one slice of the fp32 outputs at 2^31 bytes (Nq d 4)
    assert _call(fn, Nq=1 << 22) == EUNSUPPORTED
    assert _call(fn, Nq=1 << 23, d=64) == EUNSUPPORTED
    # more (b, h) slices than 2^31 - 1
    assert _call(fn, B=1 << 16, H=1 << 16, Nq=256) == EUNSUPPORTED
    # tensors past 2^31 bytes over many slices of modest size, and more slices
    # than one launch takes (65535), pass the size checks: such calls run as
    # launches over groups of slices.  They stop here at the misaligned
    # pointer, so nothing is launched.
    p = [A + j * 0x100000 for j in range(9)]
    p[0] += 4
    assert _call(fn, p, B=64, H=64, Nq=4096) == EALIGN
    assert _call(fn, p, B=256, H=256, Nq=1, Nk=1) == EALIGN
    assert _call(fn, p, B=(1 << 15) - 1, H=1 << 16, Nq=1, Nk=1) == EALIGN
    assert _call(fn, p, Nq=(1 << 22) - 1) == EALIGN


@pytest.mark.parametrize("fn", FNS)
def test_misaligned(fn):
    for i in range(8):
        p = [A + j * 0x100000 for j in range(9)]
        p[i] += 4
        assert _call(fn, p) == EALIGN, i
    p = [A + j * 0x100000 for j in range(9)]
    p[8] += 2  # lse needs 4-byte alignment
    assert _call(fn, p) == EALIGN


def test_workspace_checks():
    assert _call("attn_jvp_fwd_ws", ws=0) == EINVAL
    assert _call("attn_jvp_fwd_ws", ws_bytes=100) == EINVAL
    assert _call("attn_jvp_fwd_ws", ws=A + 0x1000000 + 16) == EALIGN


def _pack(k=A, v=A + 0x100000, tk=A + 0x200000, tv=A + 0x300000, B=1, H=1, Nk=4, d=128,
          ws=A + 0x1000000, ws_bytes=None):
    nb = ajvp.attn_jvp_workspace_bytes(max(B, 1), max(H, 1), max(Nk, 1), d)
    return ajvp.lib().attn_jvp_pack_kv(
        ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(tk), ctypes.c_void_p(tv), B, H,
        Nk, d, ctypes.c_void_p(ws), ctypes.c_size_t(nb if ws_bytes is None else ws_bytes),
        ctypes.c_void_p(0))


def _packed(ptrs=None, B=1, H=1, Nq=4, Nk=4, d=128, scale=0.1, ws=A + 0x1000000,
            ws_bytes=None):
    p = [A + i * 0x100000 for i in range(5)] if ptrs is None else ptrs  # q tq o to lse
    nb = ajvp.attn_jvp_workspace_bytes(max(B, 1), max(H, 1), max(Nk, 1), d)
    return ajvp.lib().attn_jvp_fwd_packed(
        *[ctypes.c_void_p(x) for x in p[:2]], ctypes.c_void_p(ws),
        ctypes.c_size_t(nb if ws_bytes is None else ws_bytes),
        *[ctypes.c_void_p(x) for x in p[2:]], B, H, Nq, Nk, d, ctypes.c_float(scale),
        ctypes.c_void_p(0))


def test_pack_kv_rejects_bad_arguments():
    assert _pack(k=0) == EINVAL and _pack(v=0) == EINVAL and _pack(tk=0) == EINVAL
    assert _pack(tv=0) == EINVAL and _pack(ws=0) == EINVAL
    assert _pack(ws_bytes=100) == EINVAL
    assert _pack(B=0) == EINVAL and _pack(Nk=0) == EINVAL
    assert _pack(d=96) == EUNSUPPORTED and _pack(Nk=1 << 24) == EUNSUPPORTED
    assert _pack(B=1 << 16, H=1 << 16) == EUNSUPPORTED
    assert _pack(k=A + 4) == EALIGN and _pack(v=A + 0x100000 + 8) == EALIGN
    assert _pack(tk=A + 0x200000 + 2) == EALIGN and _pack(tv=A + 0x300000 + 8) == EALIGN
    assert _pack(ws=A + 0x1000000 + 16) == EALIGN


def test_fwd_packed_rejects_bad_arguments():
    for i in range(4):  # q tq o to (lse may be NULL)
        p = [A + j * 0x100000 for j in range(5)]
        p[i] = 0
        assert _packed(p) == EINVAL, i
    assert _packed(ws=0) == EINVAL and _packed(ws_bytes=100) == EINVAL
    assert _packed(scale=float("inf")) == EINVAL and _packed(scale=float("nan")) == EINVAL
    assert _packed(Nq=0) == EINVAL
    assert _packed(d=64 + 1) == EUNSUPPORTED and _packed(Nk=1 << 24) == EUNSUPPORTED
    for i in range(4):
        p = [A + j * 0x100000 for j in range(5)]
        p[i] += 4
        assert _packed(p) == EALIGN, i
    p = [A + j * 0x100000 for j in range(5)]
    p[4] += 2
    assert _packed(p) == EALIGN
    assert _packed(ws=A + 0x1000000 + 64) == EALIGN


# ---- extended entry points ----

def _ex(ptrs=None, B=1, H=1, Nq=4, Nk=4, d=128, scale=0.1, out_dtype=0, ws=0, ws_bytes=0):
    # q k v tq tk tv o to lse tlse
    p = [A + i * 0x100000 for i in range(10)] if ptrs is None else ptrs
    return ajvp.lib().attn_jvp_fwd_ex(
        *[ctypes.c_void_p(x) for x in p], B, H, Nq, Nk, d, ctypes.c_float(scale), out_dtype,
        ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(0))


def _fwd(ptrs=None, B=1, H=1, Nq=4, Nk=4, d=128, scale=0.1, out_dtype=0, ws=0, ws_bytes=0):
    p = [A + i * 0x100000 for i in range(5)] if ptrs is None else ptrs  # q k v o lse
    return ajvp.lib().attn_fwd(
        *[ctypes.c_void_p(x) for x in p], B, H, Nq, Nk, d, ctypes.c_float(scale), out_dtype,
        ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(0))


def _merge(ptrs=None, P=2, R=8, d=128):
    p = [A + i * 0x100000 for i in range(8)] if ptrs is None else ptrs
    # lse_parts o_parts to_parts tlse_parts | lse o to tlse
    return ajvp.lib().attn_jvp_merge(*[ctypes.c_void_p(x) for x in p[:4]], P, R, d,
                                     *[ctypes.c_void_p(x) for x in p[4:]], ctypes.c_void_p(0))


def test_fwd_ex_rejects_bad_arguments():
    for i in (0, 1, 2, 6, 7):  # q k v o to are required; tangents, lse, tlse optional
        p = [A + j * 0x100000 for j in range(10)]
        p[i] = 0
        assert _ex(p) == EINVAL, i
    assert _ex(out_dtype=2) == EINVAL and _ex(out_dtype=-1) == EINVAL
    assert _ex(scale=float("nan")) == EINVAL and _ex(Nq=0) == EINVAL
    assert _ex(d=96) == EUNSUPPORTED
    for i in range(8):  # 16-byte alignment of every tensor
        p = [A + j * 0x100000 for j in range(10)]
        p[i] += 8
        assert _ex(p) == EALIGN, i
    p = [A + j * 0x100000 for j in range(10)]
    p[9] += 2  # tlse: 4-byte alignment
    assert _ex(p) == EALIGN
    # a caller workspace is checked like attn_jvp_fwd_ws's
    assert _ex(ws=A + 0x3000000, ws_bytes=100) == EINVAL
    nb = ajvp.attn_jvp_workspace_bytes(1, 1, 4, 128)
    assert _ex(ws=A + 0x3000000 + 64, ws_bytes=nb) == EALIGN


def test_fwd_ex_accepts_null_tangents_up_to_launch():
    # every combination of NULL tangents passes validation; a misaligned o stops
    # the call before anything is launched
    for mask in range(8):
        p = [A + j * 0x100000 for j in range(10)]
        for i in range(3):
            if mask >> i & 1:
                p[3 + i] = 0
        p[6] += 4
        assert _ex(p) == EALIGN, mask


def test_attn_fwd_rejects_bad_arguments():
    for i in range(4):  # q k v o (lse optional)
        p = [A + j * 0x100000 for j in range(5)]
        p[i] = 0
        assert _fwd(p) == EINVAL, i
    assert _fwd(out_dtype=3) == EINVAL and _fwd(scale=-float("inf")) == EINVAL
    assert _fwd(d=32) == EUNSUPPORTED and _fwd(B=1 << 16, H=1 << 16) == EUNSUPPORTED
    p = [A + j * 0x100000 for j in range(5)]
    p[3] += 4
    assert _fwd(p) == EALIGN


def test_merge_rejects_bad_arguments():
    for i in (0, 1, 5):  # lse_parts, o_parts, o
        p = [A + j * 0x100000 for j in range(8)]
        p[i] = 0
        assert _merge(p) == EINVAL, i
    for i in (2, 3, 6):  # the tangent arrays go together
        p = [A + j * 0x100000 for j in range(8)]
        p[i] = 0
        assert _merge(p) == EINVAL, i
    p = [A + j * 0x100000 for j in range(8)]
    p[2] = p[3] = p[6] = 0  # forward-only merge with a tlse output
    assert _merge(p) == EINVAL
    assert _merge(P=0) == EINVAL and _merge(R=0) == EINVAL
    assert _merge(d=96) == EUNSUPPORTED and _merge(P=2048) == EUNSUPPORTED
    # o_parts past 2^31 bytes: accepted (chunks of rows); stops at the misaligned pointer
    p = [A + j * 0x100000 for j in range(8)]
    p[1] += 4
    assert _merge(p, P=1024, R=1 << 20) == EALIGN
    for i in (1, 2, 5, 6):
        p = [A + j * 0x100000 for j in range(8)]
        p[i] += 8
        assert _merge(p) == EALIGN, i
    for i in (0, 3, 4, 7):
        p = [A + j * 0x100000 for j in range(8)]
        p[i] += 2
        assert _merge(p) == EALIGN, i


def _split(p=None, nsplit=0, ws=None, ws_bytes=None, **kw):
    L = ajvp.lib()
    p = [A + j * 0x100000 for j in range(10)] if p is None else p
    size = dict(B=1, H=1, Nq=4, Nk=4, d=128, scale=0.1)
    size.update(kw)
    return L.attn_jvp_fwd_splitkv(*[ctypes.c_void_p(x) for x in p], size["B"], size["H"],
                                  size["Nq"], size["Nk"], size["d"], ctypes.c_float(size["scale"]),
                                  nsplit, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes or 0),
                                  ctypes.c_void_p(0))


def test_splitkv_rejects_bad_arguments():
    for i in (0, 1, 2, 6, 7):  # q k v o to are required
        p = [A + j * 0x100000 for j in range(10)]
        p[i] = 0
        assert _split(p) == EINVAL, i
    assert _split(nsplit=-1) == EINVAL and _split(Nq=0) == EINVAL
    assert _split(scale=float("inf")) == EINVAL and _split(d=96) == EUNSUPPORTED
    for i in range(8):
        p = [A + j * 0x100000 for j in range(10)]
        p[i] += 8
        assert _split(p) == EALIGN, i
    nb = ajvp.attn_jvp_splitkv_workspace_bytes(1, 1, 4, 4, 128, 0)
    assert _split(ws=A + 0x3000000, ws_bytes=nb - 1) == EINVAL
    assert _split(ws=A + 0x3000000 + 64, ws_bytes=nb) == EALIGN


def test_splitkv_workspace_bytes():
    """Tile images (as attn_jvp_workspace_bytes, rounded up to 256 bytes), then
    with more than one range the partial O, dO (fp32 rows x d) and lse, mu
    (fp32 rows) of every range, each array rounded up to 256 bytes."""
    img = lambda B, H, Nk, d: ajvp.attn_jvp_workspace_bytes(B, H, Nk, d)
    r256 = lambda n: -(-n // 256) * 256
    def want(B, H, Nq, Nk, d, ns):
        n = r256(img(B, H, Nk, d))
        if ns > 1:
            rows = ns * B * H * Nq
            n += 2 * r256(rows * d * 4) + 2 * r256(rows * 4)
        return n
    # one range: the images alone
    assert ajvp.attn_jvp_splitkv_workspace_bytes(1, 12, 32760, 32760, 128, 1) == \
        want(1, 12, 32760, 32760, 128, 1)
    # explicit counts: 512 tiles in ranges of ceil(512 / n) tiles, so
    # ceil(512 / ceil(512 / n)) ranges (100 -> 6 tiles each -> 86 ranges)
    for n, used in ((2, 2), (3, 3), (7, 7), (100, 86), (300, 256), (5000, 512)):
        assert ajvp.attn_jvp_splitkv_workspace_bytes(1, 2, 100, 32760, 128, n) == \
            want(1, 2, 100, 32760, 128, used), n
    # automatic: the count is one of the explicit ones, 1 when the row tiles
    # fill the chip, several for few rows against many keys, and never fewer
    # than 4 tiles per range
    def auto_count(B, H, Nq, Nk, d):
        nb = ajvp.attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, 0)
        for n in range(1, 1025):
            if nb == want(B, H, Nq, Nk, d, n):
                return n
        raise AssertionError("no count matches the automatic workspace size")
    assert auto_count(1, 12, 32760, 32760, 128) == 1      # 1536 row tiles
    assert auto_count(1, 12, 32760, 512, 128) == 1        # cross-attention shape
    assert auto_count(2, 16, 4096, 4096, 128) == 1        # 512 row tiles
    # one GPU's share of the 14B shape (H = 5): the JVP kernel's 640 row tiles
    # fill 2.5 rounds of the CUs (it picks 2 ranges), the forward kernel's 320
    # tiles of 512 rows 1.25 (it picks 3); the workspace covers the larger
    assert auto_count(1, 5, 32760, 32760, 128) == 3
    assert auto_count(1, 12, 256, 32760, 128) > 8         # 12 row tiles, 512 key tiles
    assert 1 < auto_count(1, 1, 10, 512, 64) <= 2         # 8 key tiles: ranges of >= 4
    assert ajvp.attn_jvp_splitkv_workspace_bytes(1, 1, 10, 512, 64, -1) == 0


def test_grouped_workspace_bytes():
    """Calls whose tensors pass 2^31 bytes run as launches over groups of whole
    (b, h) slices (as many as keep one group's fp32 outputs under 2^31 bytes)
    that reuse one workspace in stream order: the split-KV and backward
    workspaces hold the larger of the two group sizes' needs, the tile-image
    workspace keeps one region per slice."""
    Nq, Nk, d = 32760, 100, 128
    g = (2**31 - 1) // (Nq * d * 4)
    assert g == 128
    split = lambda B, H, n: ajvp.attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, n)
    bwd = lambda B, H: ajvp.attn_bwd_workspace_bytes(B, H, Nq, Nk, d)
    for n in (0, 1, 2):
        assert split(3, 50, n) == max(split(1, g, n), split(1, 150 - g, n)) > 0, n
        assert split(1, 2 * g, n) == split(1, g, n), n
    # two ranges: a 128-slice group's partial O would pass 2^31 bytes, so that
    # group runs unsplit and the 22-slice group sets the size
    assert split(1, g, 2) == split(1, g, 1) < split(1, 22, 2) == split(3, 50, 2)
    assert bwd(3, 50) == max(bwd(1, g), bwd(1, 150 - g)) > 0
    assert ajvp.attn_jvp_workspace_bytes(3, 50, Nk, d) == 150 * ajvp.attn_jvp_workspace_bytes(1, 1, Nk, d)
    # one slice too large: no size
    assert split(1, 1, 0) > 0 and ajvp.attn_jvp_splitkv_workspace_bytes(1, 1, 1 << 22, Nk, d, 0) == 0
    assert ajvp.attn_bwd_workspace_bytes(1, 1, 1 << 22, Nk, d) == 0


def test_fwd_splitkv_rejects_bad_arguments():
    L = ajvp.lib()
    def call(p=None, nsplit=0, ws=None, ws_bytes=0, d=128, Nq=4):
        p = [A + j * 0x100000 for j in range(5)] if p is None else p  # q k v o lse
        return L.attn_fwd_splitkv(*[ctypes.c_void_p(x) for x in p], 1, 1, Nq, 4, d,
                                  ctypes.c_float(0.1), nsplit, ctypes.c_void_p(ws),
                                  ctypes.c_size_t(ws_bytes), ctypes.c_void_p(0))
    for i in range(4):  # q k v o (lse optional)
        p = [A + j * 0x100000 for j in range(5)]
        p[i] = 0
        assert call(p) == EINVAL, i
    assert call(nsplit=-2) == EINVAL and call(Nq=0) == EINVAL and call(d=96) == EUNSUPPORTED
    p = [A + j * 0x100000 for j in range(5)]
    p[3] += 8
    assert call(p) == EALIGN
    nb = ajvp.attn_jvp_splitkv_workspace_bytes(1, 1, 4, 4, 128, 0)
    assert call(ws=A + 0x3000000, ws_bytes=nb - 1) == EINVAL


def test_noalloc_validation():
    """attn_jvp_fwd_noalloc validates like attn_jvp_fwd and rejects, before any
    launch, a call whose single (b, h) slice of tile images exceeds its fixed
    device buffer (fake, never-dereferenced pointers)."""
    L = ajvp.lib()
    p = [ctypes.c_void_p(A + i * 0x100000) for i in range(9)]
    f = L.attn_jvp_fwd_noalloc
    s = ctypes.c_float(0.1)
    # 2048 key tiles x 64 KiB + the slice header > 128 MiB
    assert f(*p, 1, 1, 4, 131072, 128, s, None) == EUNSUPPORTED
    assert f(*p, 1, 1, 4, 4 * 131072, 64, s, None) == EUNSUPPORTED
    assert f(*p, 1, 1, 4, 4, 96, s, None) == EUNSUPPORTED
    assert f(*p, 0, 1, 4, 4, 128, s, None) == EINVAL
    assert f(*p, 1, 1, 4, 4, 128, ctypes.c_float(float("nan")), None) == EINVAL
    for i in range(8):
        q = list(p)
        q[i] = ctypes.c_void_p(0)
        assert f(*q, 1, 1, 4, 4, 128, s, None) == EINVAL, i
    q = list(p)
    q[2] = ctypes.c_void_p(A + 8)
    assert f(*q, 1, 1, 4, 4, 128, s, None) == EALIGN
    assert ajvp.NOALLOC_BYTES == 128 << 20
