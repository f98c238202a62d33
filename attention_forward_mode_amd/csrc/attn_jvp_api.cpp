// attn_jvp_api.cpp -- the C ABI declared in include/attn_jvp.h: argument
// validation, workspace management and dispatch to the gfx950 launchers.
// Every check runs before anything is launched, so a rejected call leaves the
// outputs untouched.
#include "attn_jvp.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "launch.hpp"

namespace {

// Every kernel addresses a tensor with 32-bit byte offsets from its base
// (buffer descriptors), so one launch's tensors stay under 2^31 bytes.  A call
// over more runs as consecutive launches over groups of whole (b, h) slices:
// the layout [B, H, N, d] keeps a group contiguous, and every slice is
// independent.  A group also holds at most 65535 slices (the pack kernels'
// grid y extent).  What stays bounded is one slice: Nq*d*4 and Nk*d*4 bytes
// (fp32 outputs, fp32 inputs) under 2^31.
constexpr int64_t kMaxTensorBytes = int64_t(1) << 31;
constexpr int64_t kMaxGroupSlices = 65535;
constexpr int64_t kMaxSlices = INT32_MAX;
constexpr int kMaxMergeParts = 1024;

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// Bytes of one (b, h) slice of each kind of tensor, and the slices per launch.
struct Slices {
  int64_t bh = 0, g = 0;  // slices in all, slices per launch (group)
  int64_t q = 0;          // Q-side input (q, tq, go): Nq*d*esize
  int64_t k = 0;          // K-side input (k, v, tk, tv): Nk*d*esize
  int64_t o = 0;          // Q-side fp32 output (o, to, gq): Nq*d*4
  int64_t ko = 0;         // K-side fp32 output (gk, gv): Nk*d*4
  int64_t r = 0;          // row scalars (lse, tlse): Nq*4
  int64_t img = 0;        // the bf16 path's tile images (workspace)
};

Slices slices(int B, int H, int Nq, int Nk, int d, int esize) {
  Slices s;
  s.bh = int64_t(B) * H;
  s.q = int64_t(Nq) * d * esize;
  s.k = int64_t(Nk) * d * esize;
  s.o = int64_t(Nq) * d * 4;
  s.ko = int64_t(Nk) * d * 4;
  s.r = int64_t(Nq) * 4;
  s.img = int64_t(ajvp::bf16_workspace_bytes(1, 1, Nk, d));
  const int64_t widest = s.o > s.ko ? s.o : s.ko;
  s.g = (kMaxTensorBytes - 1) / widest;
  if (s.g > kMaxGroupSlices) s.g = kMaxGroupSlices;
  if (s.g > s.bh) s.g = s.bh;
  return s;
}

// Runs f(s0, n) over the groups [s0, s0 + n) of s.g slices; stops at the
// first failure.
template <typename F>
hipError_t each_group(const Slices& s, F f) {
  for (int64_t s0 = 0; s0 < s.bh; s0 += s.g) {
    const hipError_t e = f(s0, static_cast<int>(s.bh - s0 < s.g ? s.bh - s0 : s.g));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// p advanced by `bytes`; NULL stays NULL (absent tangents and outputs).
template <typename T>
T* shift(T* p, int64_t bytes) {
  using C = std::conditional_t<std::is_const_v<T>, const char, char>;
  return p == nullptr ? nullptr : (T*)((C*)p + bytes);
}

// Sizes shared by every entry point: counts >= 1, d in {64, 128}, one slice
// of every tensor (inputs of esize bytes, fp32 outputs, the bf16 path's tile
// images) under 2^31 bytes, and B*H at most 2^31 - 1.
int check_sizes(int B, int H, int Nq, int Nk, int d, int esize) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_JVP_EINVAL;
  if (d != 64 && d != 128) return ATTN_JVP_EUNSUPPORTED;
  const Slices s = slices(B, H, Nq, Nk, d, esize);
  if (s.bh > kMaxSlices) return ATTN_JVP_EUNSUPPORTED;
  if (s.q >= kMaxTensorBytes || s.k >= kMaxTensorBytes || s.o >= kMaxTensorBytes ||
      s.ko >= kMaxTensorBytes || s.img >= kMaxTensorBytes)
    return ATTN_JVP_EUNSUPPORTED;
  return ATTN_JVP_OK;
}

// Any finite scale is valid: the definition holds for either sign (s < 0
// reverses the order of the logits); NaN and +-Inf are rejected.
bool bad_scale(float scale) { return !std::isfinite(scale); }

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

// One stream-ordered pool per device.  Up to kPoolKeepBytes stay cached
// between calls (the 1.3B-video shape's workspace is 403 MB, the 14B one's
// 1.3 GB); memory above that goes back to the device at the next
// synchronisation.
std::mutex g_pool_mu;
hipMemPool_t g_pool[64] = {};
constexpr uint64_t kPoolKeepBytes = uint64_t(2) << 30;

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
    uint64_t keep = kPoolKeepBytes;
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

// Split-KV and the backward pass: each group reuses the workspace from its start (images of the
// group, then its partial states, or its backward tile images and partial sums), so
// it holds the larger of the two group sizes' needs.
size_t splitkv_need(const Slices& s, int Nq, int Nk, int d, int nsplit) {
  const int64_t last = s.bh - (s.bh - 1) / s.g * s.g;
  const size_t a = ajvp::splitkv_workspace_bytes(1, int(s.g), Nq, Nk, d, nsplit);
  const size_t b = ajvp::splitkv_workspace_bytes(1, int(last), Nq, Nk, d, nsplit);
  return a > b ? a : b;
}

size_t bwd_need(const Slices& s, int Nq, int Nk, int d) {
  const int64_t last = s.bh - (s.bh - 1) / s.g * s.g;
  const size_t a = ajvp::bwd_workspace_bytes(1, int(s.g), Nq, Nk, d);
  const size_t b = ajvp::bwd_workspace_bytes(1, int(last), Nq, Nk, d);
  return a > b ? a : b;
}

bool bad_out_dtype(int t) { return t != ATTN_JVP_OUT_F32 && t != ATTN_JVP_OUT_BF16; }

}  // namespace

extern "C" {

const char* attn_jvp_strerror(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_EINVAL: return "invalid argument (null pointer, size < 1, bad scale or workspace, or size overflow)";
    case ATTN_JVP_EUNSUPPORTED: return "unsupported (head dim must be 64 or 128; one (b, h) slice of each tensor under 2^31 bytes)";
    case ATTN_JVP_EALIGN: return "misaligned pointer (tensors need 16-byte, workspace 256-byte alignment)";
    case ATTN_JVP_ELAUNCH: return "HIP launch or allocation failed";
    default: return "unknown status";
  }
}

size_t attn_jvp_workspace_bytes(int B, int H, int Nk, int d) {
  if (B < 1 || H < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  return ajvp::bf16_workspace_bytes(B, H, Nk, d);
}

// The bf16 entry points below run each group of slices with the caller's
// pointers advanced to the group's first slice; the tile-image workspace keeps
// one region per slice, so a group's images sit at s0 * (one slice's bytes).

int attn_jvp_fwd_ws(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                    const void* tv, float* o, float* to, float* lse, int B, int H, int Nq, int Nk,
                    int d, float scale, void* workspace, size_t workspace_bytes,
                    attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  rc = check_workspace(workspace, workspace_bytes, B, H, Nk, d);
  if (rc != ATTN_JVP_OK) return rc;
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  const hipError_t e = each_group(s, [&](int64_t s0, int n) {
    return ajvp::launch_bf16(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                             shift(tq, s0 * s.q), shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                             shift(o, s0 * s.o), shift(to, s0 * s.o), shift(lse, s0 * s.r), 1, n,
                             Nq, Nk, d, scale, shift(workspace, s0 * s.img),
                             reinterpret_cast<hipStream_t>(stream));
  });
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
  const Slices s = slices(B, H, 1, Nk, d, 2);
  const hipError_t e = each_group(s, [&](int64_t s0, int n) {
    return ajvp::launch_pack_kv(shift(k, s0 * s.k), shift(v, s0 * s.k), shift(tk, s0 * s.k),
                                shift(tv, s0 * s.k), 1, n, Nk, d, shift(workspace, s0 * s.img),
                                reinterpret_cast<hipStream_t>(stream));
  });
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
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  const hipError_t e = each_group(s, [&](int64_t s0, int n) {
    return ajvp::launch_bf16_packed(shift(q, s0 * s.q), shift(tq, s0 * s.q),
                                    shift(workspace, s0 * s.img), shift(o, s0 * s.o),
                                    shift(to, s0 * s.o), shift(lse, s0 * s.r), 1, n, Nq, Nk, d,
                                    scale, reinterpret_cast<hipStream_t>(stream));
  });
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

int attn_jvp_fwd(const void* q, const void* k, const void* v, const void* tq, const void* tk,
                 const void* tv, float* o, float* to, float* lse, int B, int H, int Nq, int Nk,
                 int d, float scale, attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  // one group's images, reused by the next group in stream order
  return with_workspace_n(nullptr, 0, size_t(s.g * s.img), st, [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_bf16(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                               shift(tq, s0 * s.q), shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                               shift(o, s0 * s.o), shift(to, s0 * s.o), shift(lse, s0 * s.r), 1,
                               n, Nq, Nk, d, scale, ws, st);
    });
  });
}

int attn_jvp_fwd_noalloc(const void* q, const void* k, const void* v, const void* tq,
                         const void* tk, const void* tv, float* o, float* to, float* lse, int B,
                         int H, int Nq, int Nk, int d, float scale, attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 2);
  if (rc != ATTN_JVP_OK) return rc;
  // groups of whole slices whose tile images fit the library's device buffer;
  // one slice must fit on its own
  const size_t cap = ajvp::scratch_bytes();
  Slices s = slices(B, H, Nq, Nk, d, 2);
  if (size_t(s.img) > cap) return ATTN_JVP_EUNSUPPORTED;
  const int64_t fit = int64_t(cap / size_t(s.img));
  if (s.g > fit) s.g = fit;
  void* ws = nullptr;
  if (ajvp::scratch_buffer(&ws) != hipSuccess) return ATTN_JVP_ELAUNCH;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = each_group(s, [&](int64_t s0, int n) {
    return ajvp::launch_bf16(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                             shift(tq, s0 * s.q), shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                             shift(o, s0 * s.o), shift(to, s0 * s.o), shift(lse, s0 * s.r), 1, n,
                             Nq, Nk, d, scale, ws, st);
  });
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
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
  const bool bf16 = out_dtype == ATTN_JVP_OUT_BF16;
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  const int64_t os = bf16 ? s.o / 2 : s.o;
  return with_workspace(workspace, workspace_bytes, B, H, Nk, d, st, [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_bf16_ex(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                                  shift(tq, s0 * s.q), shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                                  shift(o, s0 * os), shift(to, s0 * os), shift(lse, s0 * s.r),
                                  shift(tlse, s0 * s.r), 1, n, Nq, Nk, d, scale, bf16,
                                  shift(ws, s0 * s.img), st);
    });
  });
}

size_t attn_jvp_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int nsplit) {
  if (nsplit < 0 || check_sizes(B, H, Nq, Nk, d, 2) != ATTN_JVP_OK) return 0;
  return splitkv_need(slices(B, H, Nq, Nk, d, 2), Nq, Nk, d, nsplit);
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
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  return with_workspace_n(workspace, workspace_bytes, splitkv_need(s, Nq, Nk, d, nsplit), st,
                          [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_bf16_splitkv(shift(q, s0 * s.q), shift(k, s0 * s.k),
                                       shift(v, s0 * s.k), shift(tq, s0 * s.q),
                                       shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                                       shift(o, s0 * s.o), shift(to, s0 * s.o),
                                       shift(lse, s0 * s.r), shift(tlse, s0 * s.r), 1, n, Nq, Nk,
                                       d, scale, nsplit, ws, st);
    });
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
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  return with_workspace_n(workspace, workspace_bytes, splitkv_need(s, Nq, Nk, d, nsplit), st,
                          [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_fwd_splitkv(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                                      shift(o, s0 * s.o), shift(lse, s0 * s.r), 1, n, Nq, Nk, d,
                                      scale, nsplit, ws, st);
    });
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
  const bool bf16 = out_dtype == ATTN_JVP_OUT_BF16;
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  const int64_t os = bf16 ? s.o / 2 : s.o;
  return with_workspace(workspace, workspace_bytes, B, H, Nk, d, st, [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_fwd(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                              shift(o, s0 * os), shift(lse, s0 * s.r), 1, n, Nq, Nk, d, scale,
                              bf16, shift(ws, s0 * s.img), st);
    });
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
  if (P > kMaxMergeParts) return ATTN_JVP_EUNSUPPORTED;
  const void* al16[4] = {o_parts, to_parts, o, to};
  for (const void* p : al16)
    if (p != nullptr && misaligned(p, 16)) return ATTN_JVP_EALIGN;
  const void* al4[4] = {lse_parts, tlse_parts, lse, tlse};
  for (const void* p : al4)
    if (p != nullptr && misaligned(p, 4)) return ATTN_JVP_EALIGN;
  // chunks of rows, each under 2^31 bytes of one part's (or the output's) O
  const int64_t rows = (kMaxTensorBytes - 1) / (int64_t(d) * 4);
  for (int64_t r0 = 0; r0 < R; r0 += rows) {
    const int n = static_cast<int>(R - r0 < rows ? R - r0 : rows);
    const int64_t m = r0 * d;
    const hipError_t e = ajvp::launch_merge(
        lse_parts + r0, o_parts + m, shift(to_parts, m * 4), shift(tlse_parts, r0 * 4), P, n, d,
        shift(lse, r0 * 4), o + m, shift(to, m * 4), shift(tlse, r0 * 4),
        reinterpret_cast<hipStream_t>(stream), R);
    if (e != hipSuccess) return ATTN_JVP_ELAUNCH;
  }
  return ATTN_JVP_OK;
}

size_t attn_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (check_sizes(B, H, Nq, Nk, d, 2) != ATTN_JVP_OK) return 0;
  return bwd_need(slices(B, H, Nq, Nk, d, 2), Nq, Nk, d);
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
  // the kernels address one (b, h) slice of the workspace's tile images at a time
  if (int64_t(ajvp::bwd_workspace_bytes(1, 1, Nq, Nk, d)) >= kMaxTensorBytes)
    return ATTN_JVP_EUNSUPPORTED;
  const void* al16[8] = {q, k, v, o, go, gq, gk, gv};
  for (const void* p : al16)
    if (misaligned(p, 16)) return ATTN_JVP_EALIGN;
  if (misaligned(lse, 4)) return ATTN_JVP_EALIGN;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Slices s = slices(B, H, Nq, Nk, d, 2);
  return with_workspace_n(workspace, workspace_bytes, bwd_need(s, Nq, Nk, d), st,
                          [&](void* ws) {
    return each_group(s, [&](int64_t s0, int n) {
      return ajvp::launch_bwd(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                              shift(o, s0 * s.o), shift(go, s0 * s.q), shift(lse, s0 * s.r),
                              shift(gq, s0 * s.o), shift(gk, s0 * s.ko), shift(gv, s0 * s.ko), 1,
                              n, Nq, Nk, d, scale, ws, st);
    });
  });
}

int attn_jvp_fwd_f32(const float* q, const float* k, const float* v, const float* tq,
                     const float* tk, const float* tv, float* o, float* to, float* lse, int B,
                     int H, int Nq, int Nk, int d, float scale, attn_jvp_stream_t stream) {
  const void* in[6] = {q, k, v, tq, tk, tv};
  int rc = validate(in, 6, o, to, lse, B, H, Nq, Nk, d, scale, 4);
  if (rc != ATTN_JVP_OK) return rc;
  const Slices s = slices(B, H, Nq, Nk, d, 4);
  const hipError_t e = each_group(s, [&](int64_t s0, int n) {
    return ajvp::launch_f32(shift(q, s0 * s.q), shift(k, s0 * s.k), shift(v, s0 * s.k),
                            shift(tq, s0 * s.q), shift(tk, s0 * s.k), shift(tv, s0 * s.k),
                            shift(o, s0 * s.o), shift(to, s0 * s.o), shift(lse, s0 * s.r), 1, n,
                            Nq, Nk, d, scale, reinterpret_cast<hipStream_t>(stream));
  });
  return e == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ELAUNCH;
}

}  // extern "C"
