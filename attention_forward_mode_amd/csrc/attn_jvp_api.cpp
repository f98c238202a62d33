// attn_jvp_api.cpp -- the C ABI declared in include/attn_jvp.h: argument
// validation, workspace management and dispatch to the gfx950 launchers.
// Every check runs before anything is launched, so a rejected call leaves the
// outputs untouched.
#include "attn_jvp.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "launch.hpp"

namespace {

// Every tensor is addressed with 32-bit byte offsets from its base (buffer
// descriptors spanning the whole tensor), and B*H is the grid's y extent.
constexpr int64_t kMaxTensorBytes = int64_t(1) << 31;
constexpr int64_t kMaxSlices = 65535;
constexpr int kMaxMergeParts = 1024;

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// Sizes shared by every entry point: counts >= 1, d in {64, 128}, every
// tensor under 2^31 bytes, and one (b, h) slice of the bf16 path's tile-image
// workspace under 2^31 bytes (the kernels address it per slice).
// Grid: (ceil(Nq/256), B*H) workgroups; pack: (ceil(Nk/64), B*H).  esize is
// the input element size.
int check_sizes(int B, int H, int Nq, int Nk, int d, int esize) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_JVP_EINVAL;
  if (d != 64 && d != 128) return ATTN_JVP_EUNSUPPORTED;
  const int64_t bh = int64_t(B) * H;
  if (bh > kMaxSlices) return ATTN_JVP_EUNSUPPORTED;
  const int64_t qb = bh * Nq * d * esize, kb = bh * Nk * d * esize, ob = bh * Nq * d * 4;
  const int64_t wsb = int64_t(ajvp::bf16_workspace_bytes(1, 1, Nk, d));  // one slice
  if (qb >= kMaxTensorBytes || kb >= kMaxTensorBytes || ob >= kMaxTensorBytes ||
      wsb >= kMaxTensorBytes)
    return ATTN_JVP_EUNSUPPORTED;
  return ATTN_JVP_OK;
}

bool bad_scale(float scale) { return !(scale >= 0.0f) || std::isinf(scale); }

// Checks of the forward entry points: null pointers, sizes, scale, then
// alignment (16 bytes for tensors, 4 for lse).  `in` holds n input pointers.
int validate(const void* const* in, int n, float* o, float* to, float* lse, int B, int H,
             int Nq, int Nk, int d, float scale, int esize) {
  for (int i = 0; i < n; ++i)
    if (in[i] == nullptr) return ATTN_JVP_EINVAL;
  if (o == nullptr || to == nullptr) return ATTN_JVP_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || bad_scale(scale)) return ATTN_JVP_EINVAL;
  const int rc = check_sizes(B, H, Nq, Nk, d, esize);
  if (rc != ATTN_JVP_OK) return rc;
  for (int i = 0; i < n; ++i)
    if (misaligned(in[i], 16)) return ATTN_JVP_EALIGN;
  if (misaligned(o, 16) || misaligned(to, 16) || (lse != nullptr && misaligned(lse, 4)))
    return ATTN_JVP_EALIGN;
  return ATTN_JVP_OK;
}

// Workspace of the bf16 path: present, large enough, 256-byte aligned.
int check_workspace(const void* ws, size_t bytes, int B, int H, int Nk, int d) {
  if (ws == nullptr || bytes < ajvp::bf16_workspace_bytes(B, H, Nk, d)) return ATTN_JVP_EINVAL;
  if (misaligned(ws, 256)) return ATTN_JVP_EALIGN;
  return ATTN_JVP_OK;
}

// One stream-ordered pool per device; memory stays cached between calls.
std::mutex g_pool_mu;
hipMemPool_t g_pool[64] = {};

hipError_t device_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (g_pool[dev] == nullptr) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

// Runs `launch(ws)` with the caller's workspace (at least `need` bytes,
// 256-byte aligned) or, when it is NULL, with `need` bytes taken from the
// device pool and returned stream-ordered.
template <typename Launch>
int with_workspace_n(void* workspace, size_t workspace_bytes, size_t need, hipStream_t st,
                     Launch launch) {
  if (workspace != nullptr) {
    if (workspace_bytes < need) return ATTN_JVP_EINVAL;
    if (misaligned(workspace, 256)) return ATTN_JVP_EALIGN;
    return launch(workspace) == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
  }
  hipMemPool_t pool = nullptr;
  if (device_pool(&pool) != hipSuccess) return ATTN_JVP_ELAUNCH;
  void* ws = nullptr;
  if (hipMallocFromPoolAsync(&ws, need, pool, st) != hipSuccess) return ATTN_JVP_ELAUNCH;
  const hipError_t e = launch(ws);
  const hipError_t f = hipFreeAsync(ws, st);
  return (e == hipSuccess && f == hipSuccess) ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

// The same with the tile-image workspace of the bf16 path.
template <typename Launch>
int with_workspace(void* workspace, size_t workspace_bytes, int B, int H, int Nk, int d,
                   hipStream_t st, Launch launch) {
  return with_workspace_n(workspace, workspace_bytes, ajvp::bf16_workspace_bytes(B, H, Nk, d), st,
                          launch);
}

bool bad_out_dtype(int t) { return t != ATTN_JVP_OUT_F32 && t != ATTN_JVP_OUT_BF16; }

}  // namespace

extern "C" {

const char* attn_jvp_strerror(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_EINVAL: return "invalid argument (null pointer, size < 1, bad scale or workspace, or size overflow)";
    case ATTN_JVP_EUNSUPPORTED: return "unsupported (head dim must be 64 or 128, B*H at most 65535, each tensor under 2^31 bytes)";
    case ATTN_JVP_EALIGN: return "misaligned pointer (tensors need 16-byte, workspace 256-byte alignment)";
    case ATTN_JVP_ELAUNCH: return "HIP launch or allocation failed";
    default: return "unknown status";
  }
}

size_t attn_jvp_workspace_bytes(int B, int H, int Nk, int d) {
  if (B < 1 || H < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  return ajvp::bf16_workspace_bytes(B, H, Nk, d);
}

int attn_jvp_fwd_ws(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                    const void* tv, float* o, float* to, float* lse, int B, int H, int Nq, int Nk,
                    int d, float scale, void* workspace, size_t workspace_bytes,
                    attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  rc = check_workspace(workspace, workspace_bytes, B, H, Nk, d);
  if (rc != ATTN_JVP_OK) return rc;
  hipError_t e = ajvp::launch_bf16(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, d, scale,
                                   workspace, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_pack_kv(const void* k, const void* v, const void* tk, const void* tv, int B, int H,
                     int Nk, int d, void* workspace, size_t workspace_bytes,
                     attn_jvp_stream_t stream) {
  if (k == nullptr || v == nullptr || tk == nullptr || tv == nullptr) return ATTN_JVP_EINVAL;
  int rc = check_sizes(B, H, 1, Nk, d, 2);
  if (rc != ATTN_JVP_OK) return rc;
  rc = check_workspace(workspace, workspace_bytes, B, H, Nk, d);
  if (rc != ATTN_JVP_OK) return rc;
  if (misaligned(k, 16) || misaligned(v, 16) || misaligned(tk, 16) || misaligned(tv, 16))
    return ATTN_JVP_EALIGN;
  hipError_t e = ajvp::launch_pack_kv(k, v, tk, tv, B, H, Nk, d, workspace,
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_fwd_packed(const void* q, const void* tq, const void* workspace,
                        size_t workspace_bytes, float* o, float* to, float* lse, int B, int H,
                        int Nq, int Nk, int d, float scale, attn_jvp_stream_t stream) {
  const void* in[2] = {q, tq};
  int rc = validate(in, 2, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  rc = check_workspace(workspace, workspace_bytes, B, H, Nk, d);
  if (rc != ATTN_JVP_OK) return rc;
  hipError_t e = ajvp::launch_bf16_packed(q, tq, workspace, o, to, lse, B, H, Nq, Nk, d, scale,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_fwd(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                 const void* tv, float* o, float* to, float* lse, int B, int H, int Nq, int Nk,
                 int d, float scale, attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipMemPool_t pool = nullptr;
  if (device_pool(&pool) != hipSuccess) return ATTN_JVP_ELAUNCH;
  const size_t bytes = ajvp::bf16_workspace_bytes(B, H, Nk, d);
  void* ws = nullptr;
  if (hipMallocFromPoolAsync(&ws, bytes, pool, st) != hipSuccess) return ATTN_JVP_ELAUNCH;
  hipError_t e = ajvp::launch_bf16(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, d, scale, ws, st);
  hipError_t f = hipFreeAsync(ws, st);
  return (e == hipSuccess && f == hipSuccess) ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_fwd_ex(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                    const void* tv, void* o, void* to, float* lse, float* tlse, int B, int H,
                    int Nq, int Nk, int d, float scale, int out_dtype, void* workspace,
                    size_t workspace_bytes, attn_jvp_stream_t stream) {
  const void* in[3] = {q, k, v};
  int rc = validate(in, 3, static_cast<float*>(o), static_cast<float*>(to), lse, B, H, Nq, Nk, d,
                    scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  if (bad_out_dtype(out_dtype)) return ATTN_JVP_EINVAL;
  const void* tan[3] = {tq, tk, tv};
  for (const void* t : tan)
    if (t != nullptr && misaligned(t, 16)) return ATTN_JVP_EALIGN;
  if (tlse != nullptr && misaligned(tlse, 4)) return ATTN_JVP_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return with_workspace(workspace, workspace_bytes, B, H, Nk, d, st, [&](void* ws) {
    return ajvp::launch_bf16_ex(q, k, v, tq, tk, tv, o, to, lse, tlse, B, H, Nq, Nk, d, scale,
                                out_dtype == ATTN_JVP_OUT_BF16, ws, st);
  });
}

size_t attn_jvp_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int nsplit) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128) || nsplit < 0) return 0;
  return ajvp::splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit);
}

int attn_jvp_fwd_splitkv(const void* q, const void* k, const void* v, const void* tq,
                         const void* tk, const void* tv, float* o, float* to, float* lse,
                         float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                         int nsplit, void* workspace, size_t workspace_bytes,
                         attn_jvp_stream_t stream) {
  const void* in[3] = {q, k, v};
  int rc = validate(in, 3, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  if (nsplit < 0) return ATTN_JVP_EINVAL;
  const void* tan[3] = {tq, tk, tv};
  for (const void* t : tan)
    if (t != nullptr && misaligned(t, 16)) return ATTN_JVP_EALIGN;
  if (tlse != nullptr && misaligned(tlse, 4)) return ATTN_JVP_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t need = ajvp::splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit);
  return with_workspace_n(workspace, workspace_bytes, need, st, [&](void* ws) {
    return ajvp::launch_bf16_splitkv(q, k, v, tq, tk, tv, o, to, lse, tlse, B, H, Nq, Nk, d,
                                     scale, nsplit, ws, st);
  });
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                     int H, int Nq, int Nk, int d, float scale, int nsplit, void* workspace,
                     size_t workspace_bytes, attn_jvp_stream_t stream) {
  const void* in[3] = {q, k, v};
  if (o == nullptr) return ATTN_JVP_EINVAL;
  // validate() also wants a tangent output; o stands in for it here
  int rc = validate(in, 3, o, o, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  if (nsplit < 0) return ATTN_JVP_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t need = ajvp::splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit);
  return with_workspace_n(workspace, workspace_bytes, need, st, [&](void* ws) {
    return ajvp::launch_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, nsplit, ws, st);
  });
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Nq, int Nk, int d, float scale, int out_dtype, void* workspace,
             size_t workspace_bytes, attn_jvp_stream_t stream) {
  const void* in[3] = {q, k, v};
  if (o == nullptr) return ATTN_JVP_EINVAL;
  // validate() also wants a tangent output; o stands in for it here
  int rc = validate(in, 3, static_cast<float*>(o), static_cast<float*>(o), lse, B, H, Nq, Nk, d,
                    scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  if (bad_out_dtype(out_dtype)) return ATTN_JVP_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return with_workspace(workspace, workspace_bytes, B, H, Nk, d, st, [&](void* ws) {
    return ajvp::launch_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale,
                            out_dtype == ATTN_JVP_OUT_BF16, ws, st);
  });
}

int attn_jvp_merge(const float* lse_parts, const float* o_parts, const float* to_parts,
                   const float* tlse_parts, int P, int R, int d, float* lse, float* o, float* to,
                   float* tlse, attn_jvp_stream_t stream) {
  if (lse_parts == nullptr || o_parts == nullptr || o == nullptr) return ATTN_JVP_EINVAL;
  const bool tan = to_parts != nullptr;
  if (tan != (tlse_parts != nullptr) || tan != (to != nullptr)) return ATTN_JVP_EINVAL;
  if (!tan && tlse != nullptr) return ATTN_JVP_EINVAL;
  if (P < 1 || R < 1) return ATTN_JVP_EINVAL;
  if (d != 64 && d != 128) return ATTN_JVP_EUNSUPPORTED;
  if (P > kMaxMergeParts || int64_t(P) * R * d * 4 >= kMaxTensorBytes)
    return ATTN_JVP_EUNSUPPORTED;
  const void* al16[4] = {o_parts, to_parts, o, to};
  for (const void* p : al16)
    if (p != nullptr && misaligned(p, 16)) return ATTN_JVP_EALIGN;
  const void* al4[4] = {lse_parts, tlse_parts, lse, tlse};
  for (const void* p : al4)
    if (p != nullptr && misaligned(p, 4)) return ATTN_JVP_EALIGN;
  const hipError_t e = ajvp::launch_merge(lse_parts, o_parts, to_parts, tlse_parts, P, R, d, lse,
                                          o, to, tlse, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

size_t attn_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  return ajvp::bwd_workspace_bytes(B, H, Nq, Nk, d);
}

int attn_bwd(const void* q, const void* k, const void* v, const float* o, const void* go,
             const float* lse, float* gq, float* gk, float* gv, int B, int H, int Nq, int Nk,
             int d, float scale, void* workspace, size_t workspace_bytes,
             attn_jvp_stream_t stream) {
  const void* need[9] = {q, k, v, o, go, lse, gq, gk, gv};
  for (int i = 0; i < 9; ++i)
    if (need[i] == nullptr) return ATTN_JVP_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || bad_scale(scale)) return ATTN_JVP_EINVAL;
  int rc = check_sizes(B, H, Nq, Nk, d, 2);
  if (rc != ATTN_JVP_OK) return rc;
  // one (b, h) slice of each half of the workspace stays under 2^31 bytes
  if (int64_t(ajvp::bwd_workspace_bytes(1, 1, Nq, Nk, d)) >= kMaxTensorBytes ||
      int64_t(B) * H * Nk * d * 4 >= kMaxTensorBytes)
    return ATTN_JVP_EUNSUPPORTED;
  const void* al16[8] = {q, k, v, o, go, gq, gk, gv};
  for (const void* p : al16)
    if (misaligned(p, 16)) return ATTN_JVP_EALIGN;
  if (misaligned(lse, 4)) return ATTN_JVP_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t need_ws = ajvp::bwd_workspace_bytes(B, H, Nq, Nk, d);
  auto launch = [&](void* ws) {
    return ajvp::launch_bwd(q, k, v, o, go, lse, gq, gk, gv, B, H, Nq, Nk, d, scale, ws, st);
  };
  if (workspace != nullptr) {
    if (workspace_bytes < need_ws) return ATTN_JVP_EINVAL;
    if (misaligned(workspace, 256)) return ATTN_JVP_EALIGN;
    return launch(workspace) == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
  }
  hipMemPool_t pool = nullptr;
  if (device_pool(&pool) != hipSuccess) return ATTN_JVP_ELAUNCH;
  void* ws = nullptr;
  if (hipMallocFromPoolAsync(&ws, need_ws, pool, st) != hipSuccess) return ATTN_JVP_ELAUNCH;
  const hipError_t e = launch(ws);
  const hipError_t f = hipFreeAsync(ws, st);
  return (e == hipSuccess && f == hipSuccess) ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_fwd_f32(const float* q, const float* k, const float* v, const float* tq,
                     const float* tk, const float* tv, float* o, float* to, float* lse, int B,
                     int H, int Nq, int Nk, int d, float scale, attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 4);
  if (rc != ATTN_JVP_OK) return rc;
  hipError_t e = ajvp::launch_f32(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, d, scale,
                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

}  // extern "C"
