// attn_jvp_merge.hip -- merge of attention + JVP results computed over disjoint
// subsets of the keys (split-KV within one GPU, or the key shards of a ring /
// blockwise context-parallel layout).
//
// Softmax over the union of the key subsets, written with each subset's own
// (lse_p, O_p, dO_p, mu_p) where mu_p is the tangent of lse_p:
//   lse = log sum_p exp(lse_p),   a_p = exp(lse_p - lse)
//   O   = sum_p a_p O_p,          mu = sum_p a_p mu_p
//   dO  = sum_p a_p (dO_p + mu_p O_p) - mu O
// because dO_p + mu_p O_p is subset p's normalised sum of P (dS v + dv), and
// the full sums are the a_p-weighted subset sums.  (The operation is the one of
// the rCM record LIT-783, Anthology of the SOTA, "Key takeaways", "JVP at
// production scale", which also states that the kernel composes with context
// parallelism.)  HBM bound: one pass over the parts.
#include "cdna4.hpp"
#include "launch.hpp"

namespace ajvp {
namespace merge_path {

constexpr int kThreads = 256;

// One thread per (row, 4 consecutive columns) of R rows.  Part p of lse_p,
// tlse_p starts `stride` rows after part p - 1 (of o_p, to_p, stride * d
// elements), so a call can cover a chunk of the rows of larger parts; every
// part gets a descriptor of its own over the chunk's R rows.
__global__ __launch_bounds__(kThreads) void merge_kernel(
    const float* __restrict__ lse_p, const float* __restrict__ o_p,
    const float* __restrict__ to_p, const float* __restrict__ tlse_p, int P, int R, int d,
    int64_t stride, float* __restrict__ lse, float* __restrict__ o, float* __restrict__ to,
    float* __restrict__ tlse) {
  const bool tan = to_p != nullptr;
  const uint32_t row_bytes = (uint32_t)R * 4, mat_bytes = (uint32_t)R * (uint32_t)d * 4;
  const int64_t mat_stride = stride * d;
  const auto wl = make_rsrc(lse, row_bytes);
  const auto wo = make_rsrc(o, mat_bytes);
  const auto wto = make_rsrc(to, tan ? mat_bytes : 0u);
  const auto wtl = make_rsrc(tlse, (tan && tlse != nullptr) ? row_bytes : 0u);
  const int chunks = d / 4;
  const int64_t n = (int64_t)R * chunks;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const uint32_t row = (uint32_t)(i / chunks), c4 = (uint32_t)(i % chunks);
    float m = -INFINITY;
    for (int p = 0; p < P; ++p)
      m = fmaxf(m, buf_load4f(make_rsrc(lse_p + p * stride, row_bytes), row * 4));
    float wsum = 0.f, mu = 0.f;
    f32x4 ov = {0.f, 0.f, 0.f, 0.f}, hv = {0.f, 0.f, 0.f, 0.f};
    const uint32_t off = (row * (uint32_t)d + 4 * c4) * 4;
    for (int p = 0; p < P; ++p) {
      const float w = __expf(buf_load4f(make_rsrc(lse_p + p * stride, row_bytes), row * 4) - m);
      wsum += w;
      const f32x4 op =
          __builtin_bit_cast(f32x4, buf_load16(make_rsrc(o_p + p * mat_stride, mat_bytes), off));
      ov += w * op;
      if (tan) {
        const float mp = buf_load4f(make_rsrc(tlse_p + p * stride, row_bytes), row * 4);
        const f32x4 tp = __builtin_bit_cast(
            f32x4, buf_load16(make_rsrc(to_p + p * mat_stride, mat_bytes), off));
        mu += w * mp;
        hv += w * (tp + mp * op);
      }
    }
    const float inv = 1.0f / wsum;
    ov *= inv;
    buf_store16(wo, off, __builtin_bit_cast(u32x4, ov));
    if (tan) {
      mu *= inv;
      const f32x4 dv = hv * inv - mu * ov;
      buf_store16(wto, off, __builtin_bit_cast(u32x4, dv));
    }
    if (c4 == 0) {
      if (lse != nullptr) buf_store4(wl, row * 4, m + __logf(wsum));
      if (tan && tlse != nullptr) buf_store4(wtl, row * 4, mu);
    }
  }
}

}  // namespace merge_path

hipError_t launch_merge(const float* lse_p, const float* o_p, const float* to_p,
                        const float* tlse_p, int P, int R, int d, float* lse, float* o,
                        float* to, float* tlse, hipStream_t stream, int64_t stride) {
  using namespace merge_path;
  const int64_t n = (int64_t)R * (d / 4);
  const int64_t want = (n + kThreads - 1) / kThreads;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kThreads), 0, stream, lse_p, o_p, to_p,
                     tlse_p, P, R, d, stride > 0 ? stride : (int64_t)R, lse, o, to, tlse);
  return hipGetLastError();
}

}  // namespace ajvp
